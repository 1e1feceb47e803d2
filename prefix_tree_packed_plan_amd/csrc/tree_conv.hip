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

}  // namespace

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
