// Tree-aware causal depthwise conv1d for gfx950.
//
// "Tree Training" (arXiv 2511.00413) section 3.2 "Causal convolution",
// Eq. 11: every segment is convolved with the last W-1 inputs of its own
// path in front of it, never with the tokens that happen to precede it in the
// packed row (those belong to a sibling branch).  The tree-recurrence 0.1.0
// page ("How a tree runs") does this in one call with no per-segment
// boundaries; so does this kernel.
//
// The op is a streaming stencil (2 FLOP per byte), so it is written for HBM:
// each thread owns 16 bytes of channels (8 bf16 or 4 fp32) and walks a run of
// tokens, keeping the W-1 previous inputs in registers.  Consecutive threads
// own consecutive 16-byte chunks of one token row, so every load and store of
// a wavefront covers 1 KiB of contiguous memory.  At a segment start the
// window is refilled from the plan's history table (the packed rows of the
// W-1 path tokens before the segment), which also covers ancestors shorter
// than W-1.  Before a root the history names rows of the caller's root
// contexts, or zeros when none are given (the partition gateway of the
// same paper, appendix B.7: a cut hands the next partition its conv state).
#include <hip/hip_runtime.h>

#include "../../include/tree_gdn.h"
#include "launch.hpp"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;   // tokens per thread
constexpr int kBatch = 4;   // loads issued together (8 measured slower: fewer waves fit)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Rows are touched once (the W-1 rows re-read at tile starts aside), so the
// 16-byte accesses are non-temporal.
template <typename T, int VEC>
__device__ __forceinline__ void load_row(const T* __restrict__ p, float (&out)[VEC]) {
  if constexpr (sizeof(T) * VEC == 16) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const uint4 raw = make_uint4(v[0], v[1], v[2], v[3]);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      out[0] = __uint_as_float(raw.x);
      out[1] = __uint_as_float(raw.y);
      out[2] = __uint_as_float(raw.z);
      out[3] = __uint_as_float(raw.w);
    }
  } else if constexpr (sizeof(T) == 2 && VEC == 4) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      if constexpr (sizeof(T) == 2)
        out[i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
      else
        out[i] = reinterpret_cast<const float*>(p)[i];
    }
  }
}

template <typename T, int VEC>
__device__ __forceinline__ void store_row(T* __restrict__ p, const float (&in)[VEC]) {
  if constexpr (sizeof(T) * VEC == 16) {
    uint4 raw;
    if constexpr (sizeof(T) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(f32_to_bf16(in[2 * i])) |
               (static_cast<uint32_t>(f32_to_bf16(in[2 * i + 1])) << 16);
      raw = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      raw = make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                       __float_as_uint(in[3]));
    }
    __builtin_nontemporal_store(u32x4{raw.x, raw.y, raw.z, raw.w}, reinterpret_cast<u32x4*>(p));
  } else if constexpr (sizeof(T) == 2 && VEC == 4) {
    u32x2 v;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      v[i] = static_cast<uint32_t>(f32_to_bf16(in[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(in[2 * i + 1])) << 16);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      if constexpr (sizeof(T) == 2)
        reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16(in[i]);
      else
        reinterpret_cast<float*>(p)[i] = in[i];
    }
  }
}

// Row `src` of the path history: a packed input row (src >= 0), row -1 - src
// of the root contexts, or zeros when no contexts are given.
template <typename T, int VEC>
__device__ __forceinline__ void load_hist(const T* __restrict__ x, const T* __restrict__ ctx, int32_t src,
                                          int32_t C, int32_t c0, float (&out)[VEC]) {
  if (src >= 0) {
    load_row<T, VEC>(x + static_cast<int64_t>(src) * C + c0, out);
  } else if (ctx != nullptr) {
    load_row<T, VEC>(ctx + static_cast<int64_t>(-1 - src) * C + c0, out);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) out[e] = 0.f;
  }
}

template <typename T, int VEC, int W>
__global__ __launch_bounds__(kThreads) void tree_conv_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, int32_t n_tok, int32_t C, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ hist, int32_t n_seg, int32_t act, const T* __restrict__ ctx) {
  const int32_t c0 = (blockIdx.x * kThreads + threadIdx.x) * VEC;
  if (c0 >= C) return;
  const int32_t t0 = blockIdx.y * kTile;
  const int32_t t1 = min(t0 + kTile, n_tok);

  // Taps and bias of this thread's channels, in fp32.
  float wr[W][VEC];
  float br[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const T wv = w[static_cast<int64_t>(c0 + j) * W + i];
      if constexpr (sizeof(T) == 2)
        wr[i][j] = bf16_to_f32(__builtin_bit_cast(uint16_t, wv));
      else
        wr[i][j] = static_cast<float>(wv);
    }
    float bv = 0.f;
    if (bias != nullptr) {
      const T b = bias[c0 + j];
      if constexpr (sizeof(T) == 2)
        bv = bf16_to_f32(__builtin_bit_cast(uint16_t, b));
      else
        bv = static_cast<float>(b);
    }
    br[j] = bv;
  }

  // Segment holding t0: the largest s with seg_off[s] <= t0 (wave-uniform).
  int32_t lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (seg_off[mid] <= t0) lo = mid; else hi = mid - 1;
  }
  int32_t s = lo;
  int32_t seg_start = seg_off[s];
  int32_t next_start = seg_off[s + 1];

  // win[j] = input j+1 steps back along the path.
  constexpr int H = W - 1;
  float win[H > 0 ? H : 1][VEC];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int32_t back = j + 1;
    const int32_t pos = t0 - seg_start - back;  // path position relative to the segment
    const int32_t src = pos >= 0 ? t0 - back : hist[static_cast<int64_t>(s) * H + H + pos];
    load_hist<T, VEC>(x, ctx, src, C, c0, win[j]);
  }

  for (int32_t tb = t0; tb < t1; tb += kBatch) {
    float xv[kBatch][VEC];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (tb + u < t1) load_row<T, VEC>(x + static_cast<int64_t>(tb + u) * C + c0, xv[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int32_t t = tb + u;
      if (t >= t1) break;
      if (t == next_start) {  // a new segment: its window is its path history
        ++s;
        seg_start = next_start;
        next_start = seg_off[s + 1];
#pragma unroll
        for (int j = 0; j < H; ++j)
          load_hist<T, VEC>(x, ctx, hist[static_cast<int64_t>(s) * H + H - 1 - j], C, c0, win[j]);
      }
      float out[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float acc = br[e] + wr[W - 1][e] * xv[u][e];
#pragma unroll
        for (int j = 0; j < H; ++j) acc += wr[W - 2 - j][e] * win[j][e];
        if (act == TREE_ACT_SILU) acc = acc / (1.f + __expf(-acc));
        out[e] = acc;
      }
      store_row<T, VEC>(y + static_cast<int64_t>(t) * C + c0, out);
#pragma unroll
      for (int j = H - 1; j > 0; --j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) win[j][e] = win[j - 1][e];
      if constexpr (H > 0) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) win[0][e] = xv[u][e];
      }
    }
  }
}

// Conv context out: row (s, j) of ctx_out is history row ctx_src[s][j] (the
// W-1 path inputs ending at segment s's last token, oldest first).
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void conv_context_kernel(const T* __restrict__ x, const T* __restrict__ ctx,
                                                                T* __restrict__ out, int32_t C,
                                                                const int32_t* __restrict__ ctx_src) {
  const int32_t c0 = (blockIdx.x * kThreads + threadIdx.x) * VEC;
  if (c0 >= C) return;
  const int64_t row = blockIdx.y;  // s (W-1) + j
  float v[VEC];
  load_hist<T, VEC>(x, ctx, ctx_src[row], C, c0, v);
  store_row<T, VEC>(out + row * C + c0, v);
}

template <typename T, int VEC>
hipError_t launch_w(const ConvArgs& a, hipStream_t stream) {
  const int32_t nvec = (a.channels + VEC - 1) / VEC;
  dim3 grid((nvec + kThreads - 1) / kThreads, (a.n_tok + kTile - 1) / kTile);
  const T* x = static_cast<const T*>(a.x);
  const T* w = static_cast<const T*>(a.w);
  const T* b = static_cast<const T*>(a.bias);
  T* y = static_cast<T*>(a.y);
  const T* ctx = static_cast<const T*>(a.init_ctx);
  switch (a.width) {
    case 1: tree_conv_kernel<T, VEC, 1><<<grid, kThreads, 0, stream>>>(x, w, b, y, a.n_tok, a.channels, a.seg_off, a.hist, a.n_seg, a.act, ctx); break;
    case 2: tree_conv_kernel<T, VEC, 2><<<grid, kThreads, 0, stream>>>(x, w, b, y, a.n_tok, a.channels, a.seg_off, a.hist, a.n_seg, a.act, ctx); break;
    case 3: tree_conv_kernel<T, VEC, 3><<<grid, kThreads, 0, stream>>>(x, w, b, y, a.n_tok, a.channels, a.seg_off, a.hist, a.n_seg, a.act, ctx); break;
    case 4: tree_conv_kernel<T, VEC, 4><<<grid, kThreads, 0, stream>>>(x, w, b, y, a.n_tok, a.channels, a.seg_off, a.hist, a.n_seg, a.act, ctx); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ctx_out == nullptr || a.width < 2) return e;
  dim3 cgrid(grid.x, static_cast<unsigned>(a.n_seg) * (a.width - 1));
  conv_context_kernel<T, VEC><<<cgrid, kThreads, 0, stream>>>(x, ctx, static_cast<T*>(a.ctx_out), a.channels, a.ctx_src);
  return hipGetLastError();
}

// ---- backward -------------------------------------------------------------
//
// With z the pre-activation and dz = dy * act'(z):
//   dx[j] = sum_{d=0}^{W-1} w[W-1-d] * dz(tokens d steps after j on any path),
//   dw[i] = sum_t dz[t] * xin(t, i - (W-1)),   dbias = sum_t dz[t],
// and a root context row gets the dz of the tokens whose windows hold it.
// Past the end of its segment a token's successors are the first tokens of
// its children (or deeper, when children are shorter than W-1), so the parent
// receives the sum over all children -- the tree routing of the gradient
// ("Tree Training" section 3.2 and appendix A.2: siblings share what their
// parent hands them and their gradients add up there).  dz of every
// segment's first W-1 tokens ("heads") is computed first into a small fp32
// table; the plan lists, for every segment and distance m < W-1, the head
// tokens m steps after its end (fut) and m steps after its start (ent).

template <typename T>
__device__ __forceinline__ float to_f32(T v) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(__builtin_bit_cast(uint16_t, v));
  else return static_cast<float>(v);
}

template <typename T, int VEC, int W>
__device__ __forceinline__ void load_taps(const T* __restrict__ w, const T* __restrict__ bias, int32_t c0,
                                          float (&wr)[W][VEC], float (&br)[VEC]) {
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
#pragma unroll
    for (int i = 0; i < W; ++i) wr[i][j] = to_f32(w[static_cast<int64_t>(c0 + j) * W + i]);
    br[j] = bias != nullptr ? to_f32(bias[c0 + j]) : 0.f;
  }
}

// dz = dy * d act / d z at pre-activation z.
__device__ __forceinline__ float dact(float z, float dy, int32_t act) {
  if (act != TREE_ACT_SILU) return dy;
  const float sg = 1.f / (1.f + __expf(-z));
  return dy * sg * (1.f + z * (1.f - sg));
}

// Heads: dz of token j < min(W-1, len) of segment s, into hd[(s (W-1) + j) C + c].
template <typename T, int VEC, int W>
__global__ __launch_bounds__(kThreads) void conv_bwd_heads_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias, const T* __restrict__ dy,
    const T* __restrict__ ctx, float* __restrict__ hd, int32_t C, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ hist, int32_t act) {
  constexpr int H = W - 1;
  const int32_t c0 = (blockIdx.x * kThreads + threadIdx.x) * VEC;
  if (c0 >= C) return;
  const int32_t s = blockIdx.y / H, j = blockIdx.y % H;
  if (j >= seg_off[s + 1] - seg_off[s]) return;
  const int32_t t = seg_off[s] + j;
  float wr[W][VEC], br[VEC], xv[VEC], dv[VEC], z[VEC];
  load_taps<T, VEC, W>(w, bias, c0, wr, br);
  load_row<T, VEC>(x + static_cast<int64_t>(t) * C + c0, xv);
  load_row<T, VEC>(dy + static_cast<int64_t>(t) * C + c0, dv);
#pragma unroll
  for (int e = 0; e < VEC; ++e) z[e] = br[e] + wr[W - 1][e] * xv[e];
#pragma unroll
  for (int b = 1; b < W; ++b) {  // b steps back
    const int32_t pos = j - b;
    const int32_t src = pos >= 0 ? t - b : hist[static_cast<int64_t>(s) * H + H + pos];
    float hv[VEC];
    load_hist<T, VEC>(x, ctx, src, C, c0, hv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) z[e] += wr[W - 1 - b][e] * hv[e];
  }
  float* out = hd + static_cast<int64_t>(blockIdx.y) * C + c0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) out[e] = dact(z[e], dv[e], act);
}

// Sum of the head dz rows listed in lst[lo..hi).
template <int VEC>
__device__ __forceinline__ void head_sum(const float* __restrict__ hd, const int32_t* __restrict__ lst, int32_t lo,
                                         int32_t hi, int32_t C, int32_t c0, float (&out)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) out[e] = 0.f;
  for (int32_t k = lo; k < hi; ++k) {
    const float* r = hd + static_cast<int64_t>(lst[k]) * C + c0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) out[e] += r[e];
  }
}

// Main pass: token tiles of kTile (grid-stride over gridDim.y); per thread
// VEC channels.  dx of every token, and per-block partial sums of dw and
// dbias into part[blockIdx.y][c][0..W].
template <typename T, int VEC, int W>
__global__ __launch_bounds__(kThreads) void conv_bwd_main_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias, const T* __restrict__ dy,
    const T* __restrict__ ctx, T* __restrict__ dx, float* __restrict__ part, const float* __restrict__ hd,
    int32_t n_tok, int32_t C, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ fut_off, const int32_t* __restrict__ fut, int32_t n_seg, int32_t act) {
  constexpr int H = W - 1;
  const int32_t c0 = (blockIdx.x * kThreads + threadIdx.x) * VEC;
  if (c0 >= C) return;
  float wr[W][VEC], br[VEC];
  load_taps<T, VEC, W>(w, bias, c0, wr, br);
  float acc_w[W][VEC], acc_b[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc_b[e] = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) acc_w[i][e] = 0.f;
  }
  const int32_t n_tiles = (n_tok + kTile - 1) / kTile;
  for (int32_t tile = blockIdx.y; tile < n_tiles; tile += gridDim.y) {
    const int32_t t0 = tile * kTile, t1 = min(t0 + kTile, n_tok);
    int32_t lo = 0, hi = n_seg - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (seg_off[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    int32_t s = lo, seg_start = seg_off[s], seg_end = seg_off[s + 1];
    float win[H > 0 ? H : 1][VEC];  // win[j] = input j + 1 steps back
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int32_t pos = t0 - seg_start - (j + 1);
      const int32_t src = pos >= 0 ? t0 - (j + 1) : hist[static_cast<int64_t>(s) * H + H + pos];
      load_hist<T, VEC>(x, ctx, src, C, c0, win[j]);
    }
    float ring[W][VEC];  // ring[k] = dz of the token k steps before the current one
    const int32_t t_stop = min(t1 + H, n_tok);
    bool done = false;
    for (int32_t tb = t0; tb < t_stop && !done; tb += kBatch) {
    // x and dy of kBatch tokens in flight together (rows past a segment
    // break in the lookahead are loaded and not used; all are < n_tok).
    float xb[kBatch][VEC], db[kBatch][VEC];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (tb + u < t_stop) {
        load_row<T, VEC>(x + static_cast<int64_t>(tb + u) * C + c0, xb[u]);
        load_row<T, VEC>(dy + static_cast<int64_t>(tb + u) * C + c0, db[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int32_t t = tb + u;
      if (t >= t_stop) break;
      if (t == seg_end) {  // next segment
        if (t >= t1) {  // the lookahead stays in the tile's last segment
          done = true;
          break;
        }
        ++s;
        seg_start = seg_end;
        seg_end = seg_off[s + 1];
#pragma unroll
        for (int j = 0; j < H; ++j)
          load_hist<T, VEC>(x, ctx, hist[static_cast<int64_t>(s) * H + H - 1 - j], C, c0, win[j]);
      }
      const float(&xv)[VEC] = xb[u];
      float dz[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float z = br[e] + wr[W - 1][e] * xv[e];
#pragma unroll
        for (int j = 0; j < H; ++j) z += wr[W - 2 - j][e] * win[j][e];
        dz[e] = dact(z, db[u][e], act);
      }
      if (t < t1) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          acc_b[e] += dz[e];
          acc_w[W - 1][e] += dz[e] * xv[e];
#pragma unroll
          for (int j = 0; j < H; ++j) acc_w[W - 2 - j][e] += dz[e] * win[j][e];
        }
      }
#pragma unroll
      for (int k = W - 1; k > 0; --k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) ring[k][e] = ring[k - 1][e];
#pragma unroll
      for (int e = 0; e < VEC; ++e) ring[0][e] = dz[e];
      // dx of the token W-1 steps back: its successors all lie in this segment.
      {
        const int32_t j = t - H;
        if (j >= t0 && j >= seg_start && j < t1) {
          float o[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float a = 0.f;
#pragma unroll
            for (int d = 0; d < W; ++d) a += wr[W - 1 - d][e] * ring[H - d][e];
            o[e] = a;
          }
          store_row<T, VEC>(dx + static_cast<int64_t>(j) * C + c0, o);
        }
      }
      // At the segment's last token: the tokens whose successors run past its
      // end take the heads of its descendants.
      if (t == seg_end - 1) {
#pragma unroll
        for (int e2 = 0; e2 < H; ++e2) {  // token e2 steps before the end
          const int32_t j = t - e2;
          if (j < t0 || j < seg_start || j >= t1) continue;
          float o[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float a = 0.f;
            for (int d = 0; d <= e2; ++d) a += wr[W - 1 - d][e] * ring[e2 - d][e];
            o[e] = a;
          }
          for (int d = e2 + 1; d < W; ++d) {
            const int32_t m = d - e2 - 1;  // steps past the segment's end
            float f[VEC];
            const int64_t r = static_cast<int64_t>(s) * H + m;
            head_sum<VEC>(hd, fut, fut_off[r], fut_off[r + 1], C, c0, f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] += wr[W - 1 - d][e] * f[e];
          }
          store_row<T, VEC>(dx + static_cast<int64_t>(j) * C + c0, o);
        }
      }
#pragma unroll
      for (int j = H - 1; j > 0; --j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) win[j][e] = win[j - 1][e];
      if constexpr (H > 0) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) win[0][e] = xv[e];
      }
    }
    }
  }
  float* pp = part + (static_cast<int64_t>(blockIdx.y) * C + c0) * (W + 1);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
#pragma unroll
    for (int i = 0; i < W; ++i) pp[e * (W + 1) + i] = acc_w[i][e];
    pp[e * (W + 1) + W] = acc_b[e];
  }
}

// dw [C, W] and dbias [C] (fp32): the block partials summed in block order.
template <int W>
__global__ __launch_bounds__(kThreads) void conv_bwd_reduce_kernel(const float* __restrict__ part, int32_t n_part,
                                                                   int32_t C, float* __restrict__ dw,
                                                                   float* __restrict__ dbias) {
  const int32_t c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= C) return;
  float a[W + 1];
#pragma unroll
  for (int i = 0; i <= W; ++i) a[i] = 0.f;
  for (int32_t b = 0; b < n_part; ++b) {
    const float* p = part + (static_cast<int64_t>(b) * C + c) * (W + 1);
#pragma unroll
    for (int i = 0; i <= W; ++i) a[i] += p[i];
  }
#pragma unroll
  for (int i = 0; i < W; ++i) dw[static_cast<int64_t>(c) * W + i] = a[i];
  if (dbias != nullptr) dbias[c] = a[W];
}

// Root context rows: row m (oldest first) of root r sits k = W-1-m steps
// before the root's first token and is tap W-1-(e+k) of the token e steps
// after that first token (the head tokens listed in ent[root][e]).
template <typename T, int W>
__global__ __launch_bounds__(kThreads) void conv_bwd_ctx_kernel(
    const T* __restrict__ w, const float* __restrict__ hd, float* __restrict__ dctx, int32_t C,
    const int32_t* __restrict__ roots, const int32_t* __restrict__ ent_off, const int32_t* __restrict__ ent) {
  constexpr int H = W - 1;
  const int32_t c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= C) return;
  const int32_t r = blockIdx.y / H, m = blockIdx.y % H;
  const int32_t root = roots[r];
  const int32_t k = H - m;
  float a = 0.f;
  for (int e = 0; e + k <= H; ++e) {
    const int64_t row = static_cast<int64_t>(root) * H + e;
    float hs = 0.f;
    for (int32_t q = ent_off[row]; q < ent_off[row + 1]; ++q) hs += hd[static_cast<int64_t>(ent[q]) * C + c];
    a += to_f32(w[static_cast<int64_t>(c) * W + (H - e - k)]) * hs;
  }
  dctx[static_cast<int64_t>(blockIdx.y) * C + c] = a;
}

template <typename T, int VEC, int W>
hipError_t launch_bwd_w(const ConvBwdArgs& a, hipStream_t stream) {
  constexpr int H = W - 1;
  const int32_t nvec = (a.channels + VEC - 1) / VEC;
  const unsigned gx = (nvec + kThreads - 1) / kThreads;
  const T* x = static_cast<const T*>(a.x);
  const T* w = static_cast<const T*>(a.w);
  const T* b = static_cast<const T*>(a.bias);
  const T* dy = static_cast<const T*>(a.dy);
  const T* ctx = static_cast<const T*>(a.init_ctx);
  if (H > 0) {
    conv_bwd_heads_kernel<T, VEC, W><<<dim3(gx, a.n_seg * H), kThreads, 0, stream>>>(
        x, w, b, dy, ctx, a.heads, a.channels, a.seg_off, a.hist, a.act);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  conv_bwd_main_kernel<T, VEC, W><<<dim3(gx, a.n_part), kThreads, 0, stream>>>(
      x, w, b, dy, ctx, static_cast<T*>(a.dx), a.part, a.heads, a.n_tok, a.channels, a.seg_off, a.hist, a.fut_off,
      a.fut, a.n_seg, a.act);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned gc = (a.channels + kThreads - 1) / kThreads;
  conv_bwd_reduce_kernel<W><<<gc, kThreads, 0, stream>>>(a.part, a.n_part, a.channels, a.dw, a.dbias);
  e = hipGetLastError();
  if (e != hipSuccess || a.dinit_ctx == nullptr || H == 0) return e;
  conv_bwd_ctx_kernel<T, W><<<dim3(gc, a.n_roots * H), kThreads, 0, stream>>>(w, a.heads, a.dinit_ctx, a.channels,
                                                                            a.roots, a.ent_off, a.ent);
  return hipGetLastError();
}

template <typename T, int VEC>
hipError_t launch_bwd_v(const ConvBwdArgs& a, hipStream_t stream) {
  switch (a.width) {
    case 1: return launch_bwd_w<T, VEC, 1>(a, stream);
    case 2: return launch_bwd_w<T, VEC, 2>(a, stream);
    case 3: return launch_bwd_w<T, VEC, 3>(a, stream);
    case 4: return launch_bwd_w<T, VEC, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv_backward(const ConvBwdArgs& a, hipStream_t stream) {
  // Four channels per thread (8-byte bf16 or 16-byte fp32 accesses): the main
  // kernel keeps taps, weight-gradient sums, the dz ring and the window for
  // each channel in registers, and at 8 bf16 channels it needed 220 VGPRs
  // (two waves per SIMD) and ran 3% slower than at 4 (116 VGPRs).
  const bool bf16 = a.dtype == TREE_DTYPE_BF16;
  const uintptr_t mask = bf16 ? 7u : 15u;
  const auto aligned = [mask](const void* p) { return (reinterpret_cast<uintptr_t>(p) & mask) == 0; };
  const bool wide = (a.channels % 4 == 0) && aligned(a.x) && aligned(a.dy) && aligned(a.dx) &&
                    (a.init_ctx == nullptr || aligned(a.init_ctx));
  if (bf16) return wide ? launch_bwd_v<uint16_t, 4>(a, stream) : launch_bwd_v<uint16_t, 1>(a, stream);
  return wide ? launch_bwd_v<float, 4>(a, stream) : launch_bwd_v<float, 1>(a, stream);
}

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
  const bool bf16 = a.dtype == TREE_DTYPE_BF16;
  const int vec = bf16 ? 8 : 4;
  const auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const bool wide = (a.channels % vec == 0) && aligned(a.x) && aligned(a.y) &&
                    (a.init_ctx == nullptr || aligned(a.init_ctx)) && (a.ctx_out == nullptr || aligned(a.ctx_out));
  if (bf16) return wide ? launch_w<uint16_t, 8>(a, stream) : launch_w<uint16_t, 1>(a, stream);
  return wide ? launch_w<float, 4>(a, stream) : launch_w<float, 1>(a, stream);
}

}  // namespace tg
