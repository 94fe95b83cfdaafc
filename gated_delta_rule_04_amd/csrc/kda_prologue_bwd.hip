// Backward of the gate and normalisation prologue, gfx950.
//
// The prologue turns a layer's raw projections into KDA's inputs: q and k
// L2-normalised per token and head, g = -exp(A_log) softplus(f + dt_bias)
// (the Mamba-style gate; the Kimi-K3-Tiny-L13 card names A_log and dt_bias
// as KDA's real parameters, "The weights are real" section) and
// beta = sigmoid(b).  The miniKimiK3 card ("Architecture", KDA bullet) trains
// KDA through its chunked form, so the prologue's inputs and its two
// parameters need gradients too.  Per token row, from the gradients of the
// prepared q, k, g, beta:
//
//   dq_raw = r (dq - q (q . dq)),  r = (sum q_raw^2 + eps)^(-1/2), q = q_raw r
//   df     = dg * (-exp(A_log) sigmoid(f + dt_bias))
//   db_raw = dbeta * beta (1 - beta)
//   dA_log = sum over tokens of dg * g;  d dt_bias = sum over tokens of df
//
// Three launches around the chunked backward: prologue_prepare_kernel writes
// the prepared inputs (bf16) for it; prologue_grad_kernel applies the rules
// above and writes, per 64-token block and head, the partial sums of the two
// parameter gradients; prologue_param_reduce_kernel adds the blocks in a
// fixed order (bitwise deterministic, no atomics).
//
// Design for MI355X: both row kernels are HBM-bound elementwise passes.  A
// row of d_k channels is held by d_k / 8 consecutive lanes, 8 channels (one
// 16-byte bf16 access) each; its sums of squares and dot products reduce over
// those lanes with cross-lane shuffles.

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kPrologueBlock = 64;  // token rows of one head per gradient workgroup
typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)b[i];
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  *reinterpret_cast<u32x4p*>(p) = u32x4p{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]),
                                         pk_bf16(x[6], x[7])};  // RNE
}

// Sum over the L consecutive lanes (an aligned group) that hold one row.
template <int L>
__device__ __forceinline__ float row_total(float v) {
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The gate in natural units and its derivative with respect to f (and
// dt_bias): g = -exp(A) softplus(x), dg/dx = -exp(A) sigmoid(x), x = f + dt_bias.
// softplus in log2 units as the forward prologue takes it.
__device__ __forceinline__ void gate_and_slope(float f, float A, float bias, float& g, float& slope) {
  const float a = fast_exp2(A * kLog2e);
  const float x = f + bias;
  g = -a * softplus_log2(x * kLog2e) * (1.f / kLog2e);
  slope = -a * sigmoid_f(x);
}

template <int DK, int GG>
__global__ __launch_bounds__(256) void prologue_prepare_kernel(const bf16* __restrict__ q_raw,
                                                               const bf16* __restrict__ k_raw,
                                                               const bf16* __restrict__ f,
                                                               const bf16* __restrict__ b_raw,
                                                               const float* __restrict__ A_log,
                                                               const float* __restrict__ dt_bias, bf16* __restrict__ q,
                                                               bf16* __restrict__ k, bf16* __restrict__ g,
                                                               bf16* __restrict__ beta, long long rows, int H) {
  constexpr int L = DK / 8, NG = DK / GG;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = gid / L < rows;  // a row's L lanes are all live or all not
  const long long row = live ? gid / L : 0;
  const int l = (int)(gid % L), c0 = 8 * l, h = (int)(row % H);
  float x[8], y[8];
  load8(q_raw + row * DK + c0, x);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  float r = __builtin_amdgcn_rsqf(row_total<L>(ss) + kNormEps);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * r;
  if (live) store8(q + row * DK + c0, y);
  load8(k_raw + row * DK + c0, x);
  ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  r = __builtin_amdgcn_rsqf(row_total<L>(ss) + kNormEps);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * r;
  if (live) store8(k + row * DK + c0, y);
  if constexpr (GG == 1) {
    load8(f + row * DK + c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float slope;
      gate_and_slope(x[i], A_log[h * DK + c0 + i], dt_bias[h * DK + c0 + i], y[i], slope);
    }
    if (live) store8(g + row * DK + c0, y);
  } else if (c0 % GG == 0) {
    const int gi = c0 / GG;
    float gv, slope;
    gate_and_slope(to_f32(f[row * NG + gi]), A_log[h * NG + gi], dt_bias[h * NG + gi], gv, slope);
    if (live) g[row * NG + gi] = from_f32<bf16>(gv);
  }
  if (l == 0 && live) beta[row] = from_f32<bf16>(sigmoid_f(to_f32(b_raw[row])));
}

// Workgroup (64-token block tb, head h): 256 threads = 256 / L rows at a time.
template <int DK, int GG>
__global__ __launch_bounds__(256) void prologue_grad_kernel(
    const bf16* __restrict__ q_raw, const bf16* __restrict__ k_raw, const bf16* __restrict__ f,
    const bf16* __restrict__ b_raw, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const bf16* __restrict__ dq, const bf16* __restrict__ dk, const bf16* __restrict__ dg,
    const bf16* __restrict__ dbeta, bf16* __restrict__ dq_raw, bf16* __restrict__ dk_raw, bf16* __restrict__ df,
    bf16* __restrict__ db_raw, float* __restrict__ part_a, float* __restrict__ part_b, long long ntok, int H) {
  constexpr int L = DK / 8, NG = DK / GG, RPI = 256 / L;  // rows in flight per pass
  constexpr int NC = GG == 1 ? 8 : 1;                      // gate values per lane
  __shared__ float red[2][RPI][DK];
  const int tid = threadIdx.x, l = tid % L, slot = tid / L, c0 = 8 * l;
  const int h = blockIdx.x % H;
  const long long tb = blockIdx.x / H;
  const bool gate_lane = GG == 1 || c0 % GG == 0;
  const int gi0 = GG == 1 ? c0 : c0 / GG;  // first gate index of this lane within the row
  float Av[NC], Bv[NC], sa[NC], sb[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    Av[i] = gate_lane ? A_log[h * NG + gi0 + i] : 0.f;
    Bv[i] = gate_lane ? dt_bias[h * NG + gi0 + i] : 0.f;
    sa[i] = sb[i] = 0.f;
  }
  for (int j = slot; j < kPrologueBlock; j += RPI) {
    const long long tok = tb * kPrologueBlock + j;
    const bool live = tok < ntok;
    const long long row = (live ? tok : 0) * H + h;
    // the two normalised rows
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const bf16* xr = which ? k_raw : q_raw;
      const bf16* dy = which ? dk : dq;
      float x[8], d[8];
      load8(xr + row * DK + c0, x);
      load8(dy + row * DK + c0, d);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
      const float r = __builtin_amdgcn_rsqf(row_total<L>(ss) + kNormEps);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += x[i] * r * d[i];
      dot = row_total<L>(dot);
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = r * (d[i] - x[i] * r * dot);
      if (live) store8((which ? dk_raw : dq_raw) + row * DK + c0, d);
    }
    // the gate
    if (gate_lane) {
      float fv[NC], dgv[NC], dfv[NC];
      if constexpr (GG == 1) {
        load8(f + row * DK + c0, fv);
        load8(dg + row * DK + c0, dgv);
      } else {
        fv[0] = to_f32(f[row * NG + gi0]);
        dgv[0] = to_f32(dg[row * NG + gi0]);
      }
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        float gv, slope;
        gate_and_slope(fv[i], Av[i], Bv[i], gv, slope);
        dfv[i] = live ? dgv[i] * slope : 0.f;
        sa[i] += live ? dgv[i] * gv : 0.f;
        sb[i] += dfv[i];
      }
      if (live) {
        if constexpr (GG == 1)
          store8(df + row * DK + c0, dfv);
        else
          df[row * NG + gi0] = from_f32<bf16>(dfv[0]);
      }
    }
    if (l == 0 && live) {
      const float bt = sigmoid_f(to_f32(b_raw[row]));
      db_raw[row] = from_f32<bf16>(to_f32(dbeta[row]) * bt * (1.f - bt));
    }
  }
  // the block's parameter-gradient sums: the row slots in a fixed order
  if (gate_lane) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      red[0][slot][gi0 + i] = sa[i];
      red[1][slot][gi0 + i] = sb[i];
    }
  }
  __syncthreads();
  for (int c = tid; c < 2 * NG; c += 256) {
    const int which = c / NG, gi = c % NG;
    float s = 0.f;
    for (int r = 0; r < RPI; ++r) s += red[which][r][gi];
    (which ? part_b : part_a)[(tb * H + h) * NG + gi] = s;
  }
}

// dA_log, d dt_bias [H][NG]: the blocks' partial sums.  A workgroup owns 64
// consecutive outputs; its four wavefronts sum every fourth block each (in
// block order, coalesced across the 64 outputs), then the four partial sums
// are added in wavefront order: a fixed order, so the result is bitwise
// deterministic.
__global__ __launch_bounds__(256) void prologue_param_reduce_kernel(const float* __restrict__ part_a,
                                                                    const float* __restrict__ part_b,
                                                                    float* __restrict__ dA_log,
                                                                    float* __restrict__ ddt_bias, long long nblk,
                                                                    int HG) {
  __shared__ float red[2][4][64];
  const int lane = threadIdx.x % 64, grp = threadIdx.x / 64;
  const int i = blockIdx.x * 64 + lane;
  float a = 0.f, b = 0.f;
  if (i < HG) {
    for (long long t = grp; t < nblk; t += 4) {
      a += part_a[t * HG + i];
      b += part_b[t * HG + i];
    }
  }
  red[0][grp][lane] = a;
  red[1][grp][lane] = b;
  __syncthreads();
  if (grp == 0 && i < HG) {
    dA_log[i] = ((red[0][0][lane] + red[0][1][lane]) + red[0][2][lane]) + red[0][3][lane];
    ddt_bias[i] = ((red[1][0][lane] + red[1][1][lane]) + red[1][2][lane]) + red[1][3][lane];
  }
}

template <int DK, int GG>
hipError_t prologue_prepare_t(const PrologueBwdArgs& a, hipStream_t s) {
  const long long rows = a.ntok * a.H;
  const long long threads = rows * (DK / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL((prologue_prepare_kernel<DK, GG>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     a.q_raw, a.k_raw, a.f, a.b_raw, a.A_log, a.dt_bias, a.q, a.k, a.g, a.beta, rows, a.H);
  return hipGetLastError();
}

template <int DK, int GG>
hipError_t prologue_grad_t(const PrologueBwdArgs& a, hipStream_t s) {
  const long long nblk = (a.ntok + kPrologueBlock - 1) / kPrologueBlock;
  if (nblk > 0) {
    hipLaunchKernelGGL((prologue_grad_kernel<DK, GG>), dim3((unsigned)(nblk * a.H)), dim3(256), 0, s, a.q_raw,
                       a.k_raw, a.f, a.b_raw, a.A_log, a.dt_bias, a.dq, a.dk, a.dg, a.dbeta, a.dq_raw, a.dk_raw, a.df,
                       a.db_raw, a.part_a, a.part_b, a.ntok, a.H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int HG = a.H * (DK / GG);
  hipLaunchKernelGGL(prologue_param_reduce_kernel, dim3((HG + 63) / 64), dim3(256), 0, s, a.part_a, a.part_b,
                     a.dA_log, a.ddt_bias, nblk, HG);
  return hipGetLastError();
}

}  // namespace

long long prologue_bwd_blocks(long long ntok) { return (ntok + kPrologueBlock - 1) / kPrologueBlock; }

hipError_t launch_prologue_prepare(int Dk, int g_group, const PrologueBwdArgs& a, hipStream_t s) {
  if (Dk == 128) return g_group == 1 ? prologue_prepare_t<128, 1>(a, s) : prologue_prepare_t<128, 64>(a, s);
  if (Dk == 64) return g_group == 1 ? prologue_prepare_t<64, 1>(a, s) : prologue_prepare_t<64, 64>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prologue_grad(int Dk, int g_group, const PrologueBwdArgs& a, hipStream_t s) {
  if (Dk == 128) return g_group == 1 ? prologue_grad_t<128, 1>(a, s) : prologue_grad_t<128, 64>(a, s);
  if (Dk == 64) return g_group == 1 ? prologue_grad_t<64, 1>(a, s) : prologue_grad_t<64, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kda
