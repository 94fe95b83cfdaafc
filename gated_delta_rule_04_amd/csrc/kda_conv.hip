// Short causal depthwise convolution along the token axis, with document
// reset, gfx950.
//
// The miniKimiK3 card ("Limitations") says order information reaches the
// model only through KDA's decay and short convolutions plus the causal mask;
// the Mini-K3-1H-mamba2 README (packed-document paragraph) resets convolution
// history at every document boundary.  Per channel c and token t of a
// sequence (or document) starting at s:
//
//   y[t][c] = sum_{w=0}^{W-1} weight[c][w] * x[t - (W-1) + w][c]
//
// with positions before s read from the initial conv state (the W-1 inputs
// that preceded the sequence) or zero.  No bias, no activation; fp32
// accumulation.
//
// Design for MI355X: the step is HBM-bound (one read of x, one write of y).
// A thread owns 8 channels (one 16-byte access per token in bf16) and a run of
// 256 consecutive tokens, keeping the W-wide window in registers, so every
// input is read once (plus W-1 history rows per run).  Inside a document the
// run advances 8 tokens at a time with all 8 loads issued together; y is
// written with non-temporal stores.  Adjacent threads own adjacent channel
// groups, so a wavefront's accesses are contiguous.

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kConvRun = 256;  // tokens per thread

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x8 load8(const bf16* p) {
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(p);
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (float)b[i];
  return r;
}
__device__ __forceinline__ f32x8 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void store8(bf16* p, const f32x8& x) {
  const u32x4v b = {pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]), pk_bf16(x[6], x[7])};  // RNE
  __builtin_nontemporal_store(b, reinterpret_cast<u32x4v*>(p));  // written once
}
__device__ __forceinline__ void store8(float* p, const f32x8& x) {
  *reinterpret_cast<f32x4*>(p) = __builtin_shufflevector(x, x, 0, 1, 2, 3);
  *reinterpret_cast<f32x4*>(p + 4) = __builtin_shufflevector(x, x, 4, 5, 6, 7);
}

// Sequence n of the call: [start, end) in flattened token coordinates.
__device__ __forceinline__ void seq_range(const int* cu, int n, int B, int T, int& s, int& e) {
  if (cu) {
    const int a = min(max(cu[n], 0), T);
    s = a;
    e = min(max(cu[n + 1], a), T);
  } else {
    s = n * T;
    e = s + T;
  }
}

// The sequence holding token t: the last n with start(n) <= t (cu
// non-decreasing); a token past every sequence maps to num_seqs - 1.
__device__ __forceinline__ int seq_of(const int* cu, int num_seqs, int T, int t) {
  if (!cu) return t / T;
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min(max(cu[mid], 0), T) <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// History value at position p (< s) of sequence n: conv0 row p - s + W - 1.
template <typename T, int W>
__device__ __forceinline__ f32x8 history(const T* conv0, int n, int C, int ch, int row) {
  if (!conv0 || row < 0) return f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  return load8(conv0 + ((size_t)n * (W - 1) + row) * C + ch);
}

}  // namespace

template <typename T, int W>
__global__ __launch_bounds__(256) void short_conv_fwd_kernel(const T* __restrict__ x, const T* __restrict__ weight,
                                                             const T* __restrict__ conv0, T* __restrict__ y,
                                                             const int* __restrict__ cu, int num_seqs, int B,
                                                             int T_, int C) {
  const int CG = C / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long ntok = (long long)B * T_;
  const int cg = (int)(gid % CG);
  const long long run = gid / CG;
  const long long t0l = run * kConvRun;
  if (t0l >= ntok) return;
  const int t0 = (int)t0l, t1 = (int)min(t0l + kConvRun, ntok);
  const int ch = 8 * cg;

  f32x8 wg[W];  // weights of this thread's channels
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int w = 0; w < W; ++w) wg[w][c] = to_f32(weight[(size_t)(ch + c) * W + w]);

  int n = seq_of(cu, num_seqs, T_, t0), s, e;
  seq_range(cu, n, B, T_, s, e);
  f32x8 win[W];  // win[0..W-2]: the W-1 inputs before the current token
#pragma unroll
  for (int h = 0; h < W - 1; ++h) {
    const int p = t0 - (W - 1) + h;
    win[h] = p >= s ? load8(x + (size_t)p * C + ch) : history<T, W>(conv0, n, C, ch, p - s + W - 1);
  }
  int t = t0;
  // Fast path: groups of 8 tokens inside the current sequence, all 8 loads
  // issued before any arithmetic so that they are in flight together.
  for (; t + 8 <= t1 && t + 8 <= e; t += 8) {
    f32x8 xin[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) xin[u] = load8(x + (size_t)(t + u) * C + ch);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      win[W - 1] = xin[u];
      f32x8 acc = wg[0] * win[0];
#pragma unroll
      for (int w = 1; w < W; ++w) acc += wg[w] * win[w];
      store8(y + (size_t)(t + u) * C + ch, acc);
#pragma unroll
      for (int w = 0; w < W - 1; ++w) win[w] = win[w + 1];
    }
  }
  for (; t < t1; ++t) {
    if (t >= e && n + 1 < num_seqs) {  // the next non-empty sequence starts here
      do {
        ++n;
        seq_range(cu, n, B, T_, s, e);
      } while (t >= e && n + 1 < num_seqs);
#pragma unroll
      for (int h = 0; h < W - 1; ++h) {
        const int p = t - (W - 1) + h;
        win[h] = p >= s ? load8(x + (size_t)p * C + ch) : history<T, W>(conv0, n, C, ch, p - s + W - 1);
      }
    }
    win[W - 1] = load8(x + (size_t)t * C + ch);
    f32x8 acc = wg[0] * win[0];
#pragma unroll
    for (int w = 1; w < W; ++w) acc += wg[w] * win[w];
    store8(y + (size_t)t * C + ch, acc);
#pragma unroll
    for (int w = 0; w < W - 1; ++w) win[w] = win[w + 1];
  }
}

// Each sequence's last W-1 inputs.
template <typename T, int W>
__global__ __launch_bounds__(256) void short_conv_final_kernel(const T* __restrict__ x, const T* __restrict__ conv0,
                                                               T* __restrict__ conv_final, const int* __restrict__ cu,
                                                               int num_seqs, int B, int T_, int C) {
  const int CG = C / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)num_seqs * CG) return;
  const int cg = (int)(gid % CG), n = (int)(gid / CG), ch = 8 * cg;
  int s, e;
  seq_range(cu, n, B, T_, s, e);
#pragma unroll
  for (int h = 0; h < W - 1; ++h) {
    const int p = e - (W - 1) + h;
    const f32x8 v = p >= s ? load8(x + (size_t)p * C + ch) : history<T, W>(conv0, n, C, ch, p - s + W - 1);
    store8(conv_final + ((size_t)n * (W - 1) + h) * C + ch, v);
  }
}

// One decode step, state in place.
template <typename T, int W>
__global__ __launch_bounds__(256) void short_conv_step_kernel(const T* __restrict__ x, const T* __restrict__ weight,
                                                              T* __restrict__ state, T* __restrict__ y, int N,
                                                              int C) {
  const int CG = C / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)N * CG) return;
  const int cg = (int)(gid % CG), n = (int)(gid / CG), ch = 8 * cg;
  f32x8 win[W];
#pragma unroll
  for (int h = 0; h < W - 1; ++h) win[h] = load8(state + ((size_t)n * (W - 1) + h) * C + ch);
  win[W - 1] = load8(x + (size_t)n * C + ch);
  f32x8 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < W; ++w) {
    f32x8 wg;
#pragma unroll
    for (int c = 0; c < 8; ++c) wg[c] = to_f32(weight[(size_t)(ch + c) * W + w]);
    acc += wg * win[w];
  }
  store8(y + (size_t)n * C + ch, acc);
#pragma unroll
  for (int h = 0; h < W - 1; ++h) store8(state + ((size_t)n * (W - 1) + h) * C + ch, win[h + 1]);
}

// ---------------------------------------------------------------------------
// Backward.  With L = <dy, y> + <dfinal, conv_final>, per channel, for a
// token t of a sequence [s, e):
//   dx[t]  = sum_{u=0}^{W-1} weight[W-1-u] dy[t+u]  (terms with t+u >= e absent)
//            + dfinal[t - (e - (W-1))]              (for t >= e - (W-1))
//   dw[j] += dy[t] x[t - (W-1) + j]                  (history / zeros before s)
//   dconv0[row] for the history position p = s - (W-1) + row: the dx sum at p.
// A thread owns 8 channels and a run of 256 tokens, with a window of the
// next W dy rows in registers (the forward's window, mirrored) and the last
// W-1 x rows for dw; its dw sums go to a per-run partial that a second
// kernel adds in run order (bitwise deterministic).
// ---------------------------------------------------------------------------
template <typename T, int W>
__global__ __launch_bounds__(256) void short_conv_bwd_kernel(const T* __restrict__ x, const T* __restrict__ weight,
                                                             const T* __restrict__ conv0, const T* __restrict__ dy,
                                                             const T* __restrict__ dfinal, T* __restrict__ dx,
                                                             float* __restrict__ part, const int* __restrict__ cu,
                                                             int num_seqs, int B, int T_, int C) {
  const int CG = C / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long ntok = (long long)B * T_;
  const int cg = (int)(gid % CG);
  const long long run = gid / CG;
  const long long t0l = run * kConvRun;
  if (t0l >= ntok) return;
  const int t0 = (int)t0l, t1 = (int)min(t0l + kConvRun, ntok);
  const int ch = 8 * cg;
  const f32x8 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x8 wg[W], dw[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    dw[w] = zero;
#pragma unroll
    for (int c = 0; c < 8; ++c) wg[w][c] = to_f32(weight[(size_t)(ch + c) * W + w]);
  }
  int n = seq_of(cu, num_seqs, T_, t0), s, e;
  seq_range(cu, n, B, T_, s, e);
  f32x8 dwin[W], xwin[W];  // dwin[u] = dy[t + u]; xwin[j] = x[t - (W-1) + j]
  auto seed = [&](int t) {
#pragma unroll
    for (int u = 0; u < W; ++u) dwin[u] = t + u < e ? load8(dy + (size_t)(t + u) * C + ch) : zero;
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int p = t - (W - 1) + j;
      xwin[j] = p >= s ? load8(x + (size_t)p * C + ch) : history<T, W>(conv0, n, C, ch, p - s + W - 1);
    }
  };
  seed(t0);
  int t = t0;
  // Fast path: groups of NG tokens whose look-ahead stays inside the current
  // sequence and whose dx needs no final-state term; the x and dy loads of a
  // group are issued together.  Pairs for W <= 5 (K3 width, W = 4: 0.62 ->
  // 0.53 ms); wider windows keep one token at a time, where the extra
  // registers of a group cost more than its loads in flight gain.
  constexpr int NG = W <= 5 ? 2 : 1;
  for (; t + NG <= t1 && t + NG + W <= e; t += NG) {
    f32x8 xin[NG], dyin[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      xin[u] = load8(x + (size_t)(t + u) * C + ch);
      dyin[u] = load8(dy + (size_t)(t + u + W) * C + ch);
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      xwin[W - 1] = xin[u];
      f32x8 acc = wg[W - 1] * dwin[0];
#pragma unroll
      for (int v = 1; v < W; ++v) acc += wg[W - 1 - v] * dwin[v];
      store8(dx + (size_t)(t + u) * C + ch, acc);
#pragma unroll
      for (int j = 0; j < W; ++j) dw[j] += dwin[0] * xwin[j];
#pragma unroll
      for (int v = 0; v < W - 1; ++v) dwin[v] = dwin[v + 1];
      dwin[W - 1] = dyin[u];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) xwin[j] = xwin[j + 1];
    }
  }
  for (; t < t1; ++t) {
    if (t >= e && n + 1 < num_seqs) {  // the next non-empty sequence starts here
      do {
        ++n;
        seq_range(cu, n, B, T_, s, e);
      } while (t >= e && n + 1 < num_seqs);
      seed(t);
    }
    xwin[W - 1] = load8(x + (size_t)t * C + ch);
    f32x8 acc = wg[W - 1] * dwin[0];
#pragma unroll
    for (int u = 1; u < W; ++u) acc += wg[W - 1 - u] * dwin[u];
    if (dfinal && W > 1 && t >= e - (W - 1)) acc += load8(dfinal + ((size_t)n * (W - 1) + t - (e - (W - 1))) * C + ch);
    store8(dx + (size_t)t * C + ch, acc);
#pragma unroll
    for (int j = 0; j < W; ++j) dw[j] += dwin[0] * xwin[j];
#pragma unroll
    for (int u = 0; u < W - 1; ++u) dwin[u] = dwin[u + 1];
    dwin[W - 1] = t + W < e ? load8(dy + (size_t)(t + W) * C + ch) : zero;
#pragma unroll
    for (int j = 0; j < W - 1; ++j) xwin[j] = xwin[j + 1];
  }
#pragma unroll
  for (int j = 0; j < W; ++j) {
    float* pr = part + ((size_t)run * W + j) * C + ch;
    *reinterpret_cast<f32x4*>(pr) = __builtin_shufflevector(dw[j], dw[j], 0, 1, 2, 3);
    *reinterpret_cast<f32x4*>(pr + 4) = __builtin_shufflevector(dw[j], dw[j], 4, 5, 6, 7);
  }
}

// dconv0 of each sequence: the dx sums at its W-1 history positions.
template <typename T, int W>
__global__ __launch_bounds__(256) void short_conv_bwd_state_kernel(const T* __restrict__ weight,
                                                                   const T* __restrict__ dy,
                                                                   const T* __restrict__ dfinal,
                                                                   T* __restrict__ dconv0, const int* __restrict__ cu,
                                                                   int num_seqs, int B, int T_, int C) {
  const int CG = C / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)num_seqs * CG) return;
  const int cg = (int)(gid % CG), n = (int)(gid / CG), ch = 8 * cg;
  int s, e;
  seq_range(cu, n, B, T_, s, e);
  f32x8 wg[W];
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int c = 0; c < 8; ++c) wg[w][c] = to_f32(weight[(size_t)(ch + c) * W + w]);
#pragma unroll
  for (int row = 0; row < W - 1; ++row) {
    const int p = s - (W - 1) + row;
    f32x8 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const int t = p + u;
      if (t >= s && t < e) acc += wg[W - 1 - u] * load8(dy + (size_t)t * C + ch);
    }
    // the final state holds position p when the sequence is shorter than W-1
    if (dfinal && p >= e - (W - 1)) acc += load8(dfinal + ((size_t)n * (W - 1) + p - (e - (W - 1))) * C + ch);
    store8(dconv0 + ((size_t)n * (W - 1) + row) * C + ch, acc);
  }
}

// dweight [C][W] (fp32): the per-run partial sums added in run order.
__global__ __launch_bounds__(256) void short_conv_bwd_weight_kernel(const float* __restrict__ part,
                                                                    float* __restrict__ dweight, long long runs, int C,
                                                                    int W) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // i = j * C + c
  if (i >= C * W) return;
  const int j = i / C, c = i % C;
  float a = 0.f;
  for (long long r = 0; r < runs; ++r) a += part[(r * W + j) * C + c];
  dweight[(size_t)c * W + j] = a;
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <typename T, int W>
static hipError_t conv_fwd_w(const void* x, const void* weight, const void* conv0, void* y, void* conv_final,
                             const int* cu, int num_seqs, int B, int T_, int C, hipStream_t s) {
  const long long ntok = (long long)B * T_;
  const long long runs = (ntok + kConvRun - 1) / kConvRun;
  const long long threads = runs * (C / 8);
  if (threads > 0) {
    hipLaunchKernelGGL((short_conv_fwd_kernel<T, W>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       (const T*)x, (const T*)weight, (const T*)conv0, (T*)y, cu, num_seqs, B, T_, C);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (conv_final && W > 1 && num_seqs > 0) {
    const long long ft = (long long)num_seqs * (C / 8);
    hipLaunchKernelGGL((short_conv_final_kernel<T, W>), dim3((unsigned)((ft + 255) / 256)), dim3(256), 0, s,
                       (const T*)x, (const T*)conv0, (T*)conv_final, cu, num_seqs, B, T_, C);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int W>
static hipError_t conv_step_w(const void* x, const void* weight, void* state, void* y, int N, int C, hipStream_t s) {
  const long long threads = (long long)N * (C / 8);
  hipLaunchKernelGGL((short_conv_step_kernel<T, W>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const T*)x, (const T*)weight, (T*)state, (T*)y, N, C);
  return hipGetLastError();
}

template <typename T, int W>
static hipError_t conv_bwd_w(const void* x, const void* weight, const void* conv0, const void* dy, const void* dfinal,
                             void* dx, float* dweight, void* dconv0, float* part, const int* cu, int num_seqs, int B,
                             int T_, int C, hipStream_t s) {
  const long long ntok = (long long)B * T_;
  const long long runs = (ntok + kConvRun - 1) / kConvRun;
  const long long threads = runs * (C / 8);
  if (threads > 0) {
    hipLaunchKernelGGL((short_conv_bwd_kernel<T, W>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       (const T*)x, (const T*)weight, (const T*)conv0, (const T*)dy, (const T*)dfinal, (T*)dx, part,
                       cu, num_seqs, B, T_, C);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(short_conv_bwd_weight_kernel, dim3((unsigned)((C * W + 255) / 256)), dim3(256), 0, s, part,
                     dweight, runs, C, W);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dconv0 && W > 1 && num_seqs > 0) {
    const long long ft = (long long)num_seqs * (C / 8);
    hipLaunchKernelGGL((short_conv_bwd_state_kernel<T, W>), dim3((unsigned)((ft + 255) / 256)), dim3(256), 0, s,
                       (const T*)weight, (const T*)dy, (const T*)dfinal, (T*)dconv0, cu, num_seqs, B, T_, C);
    err = hipGetLastError();
  }
  return err;
}

long long short_conv_bwd_runs(long long ntok) { return (ntok + kConvRun - 1) / kConvRun; }

#define KDA_CONV_SWITCH(W_, CALL) \
  switch (W_) {                   \
    case 1: return CALL(1);       \
    case 2: return CALL(2);       \
    case 3: return CALL(3);       \
    case 4: return CALL(4);       \
    case 5: return CALL(5);       \
    case 6: return CALL(6);       \
    case 7: return CALL(7);       \
    case 8: return CALL(8);       \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_short_conv_fwd(bool bf16_io, const void* x, const void* weight, const void* conv0, void* y,
                                 void* conv_final, const int* cu, int num_seqs, int B, int T, int C, int W,
                                 hipStream_t s) {
  if (bf16_io) {
#define CALL(w) conv_fwd_w<bf16, w>(x, weight, conv0, y, conv_final, cu, num_seqs, B, T, C, s)
    KDA_CONV_SWITCH(W, CALL)
#undef CALL
  }
#define CALL(w) conv_fwd_w<float, w>(x, weight, conv0, y, conv_final, cu, num_seqs, B, T, C, s)
  KDA_CONV_SWITCH(W, CALL)
#undef CALL
}

hipError_t launch_short_conv_step(bool bf16_io, const void* x, const void* weight, void* state, void* y, int N,
                                  int C, int W, hipStream_t s) {
  if (bf16_io) {
#define CALL(w) conv_step_w<bf16, w>(x, weight, state, y, N, C, s)
    KDA_CONV_SWITCH(W, CALL)
#undef CALL
  }
#define CALL(w) conv_step_w<float, w>(x, weight, state, y, N, C, s)
  KDA_CONV_SWITCH(W, CALL)
#undef CALL
}


hipError_t launch_short_conv_bwd(bool bf16_io, const void* x, const void* weight, const void* conv0, const void* dy,
                                 const void* dfinal, void* dx, float* dweight, void* dconv0, float* part,
                                 const int* cu, int num_seqs, int B, int T, int C, int W, hipStream_t s) {
  if (bf16_io) {
#define CALL(w) conv_bwd_w<bf16, w>(x, weight, conv0, dy, dfinal, dx, dweight, dconv0, part, cu, num_seqs, B, T, C, s)
    KDA_CONV_SWITCH(W, CALL)
#undef CALL
  }
#define CALL(w) conv_bwd_w<float, w>(x, weight, conv0, dy, dfinal, dx, dweight, dconv0, part, cu, num_seqs, B, T, C, s)
  KDA_CONV_SWITCH(W, CALL)
#undef CALL
}
#undef KDA_CONV_SWITCH

}  // namespace kda
