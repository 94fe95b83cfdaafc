// KDA recurrent decode step (one token per sequence, every head), gfx950.
//
// The decode form of the miniKimiK3 card's Kimi Delta Attention bullet
// ("Architecture" section): a fixed d_k x d_v state per head, constant cost
// per token.  Per (sequence, head), with alpha = exp(g):
//
//     S'  = Diag(alpha) S                      decay (key channels = rows)
//     e   = S'^T k,  y = S'^T q                 two reductions over the rows
//     u   = beta (v - e)                        delta-rule correction
//     o   = y + (q . k) u                       = (S' + k u^T)^T q
//     S  <- S' + k u^T                          written back in place
//
// The step is bound by HBM: the float32 state is read once and written once
// (2 * 4 * Dk * Dv bytes per head); everything else is a few hundred bytes.
// One workgroup of 512 threads owns one (sequence, head) state and keeps it in
// registers between the read and the write, so the identity for o needs no
// second pass.  Each thread owns 4 adjacent value columns (one 16-byte load
// per row) and a strided set of rows; a wavefront's loads cover whole
// contiguous rows, so every access is a fully coalesced 16-byte load/store.
// The state is read with non-temporal loads: it is streamed once per step and
// the pool is far larger than the caches.  It is written back with
// non-temporal stores except by the last eighth of the grid, whose ordinary
// stores stay in the 256 MB memory-side cache and drain under the next kernel:
// at N=256, H=96, d=128 (1.6 GB of fp32 state) this runs 64 back-to-back steps
// at 0.557 ms each, against 0.602 ms with ordinary stores throughout and 0.567
// ms with non-temporal stores throughout, and keeps a step that alternates
// with the prefill at 0.553 ms (0.576 ms with non-temporal stores throughout).
// The two column reductions run through cross-lane shuffles and an LDS
// exchange between the 8 wavefronts.
//
// Serving form: the states live in a pool and sequence n uses slot slots[n]
// (the state pool that bounds concurrency in the K3-Tiny-L13 card's serving
// notes, with the state dtype as a knob).  A slot outside the pool marks an
// inactive sequence: its output row is zero and no state is touched.  A bf16
// or fp16 pool is widened to fp32 for the step and rounded to nearest even
// after it.  An optional output gate (the Mini-K3-1H cards list output gates
// among the family's operators) scales the output by sigmoid(z), one logit
// per value channel; it never reaches the state.
//
// Prologue form (PRO): q and k arrive raw and are L2-normalised here, g holds
// the gate logits f (g = -exp(A_log) softplus(f + dt_bias)) and beta the
// logits b (beta = sigmoid(b)).  The inverse norms enter as scalar factors of
// the two reductions and of the write, so the state stream is unchanged.

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Four consecutive state values (fp32: one 16-byte access; bf16: one 8-byte
// access), streamed with non-temporal loads.
__device__ __forceinline__ f32x4 load_state4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ f32x4 load_state4(const bf16* p) {
  const bf16x4 b = __builtin_bit_cast(bf16x4, __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p)));
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
__device__ __forceinline__ f32x4 load_state4(const f16* p) {
  const f16x4 h = __builtin_bit_cast(f16x4, __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p)));
  return __builtin_convertvector(h, f32x4);
}
// Write-back of four state values; NT selects non-temporal stores.
template <bool NT>
__device__ __forceinline__ void store_state4(float* p, const f32x4& x) {
  if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
  else *reinterpret_cast<f32x4*>(p) = x;
}
template <bool NT>
__device__ __forceinline__ void store_state4(bf16* p, const f32x4& x) {
  const u32x2v b = __builtin_bit_cast(u32x2v, to_bf16x4(x));  // RNE
  if constexpr (NT) __builtin_nontemporal_store(b, reinterpret_cast<u32x2v*>(p));
  else *reinterpret_cast<u32x2v*>(p) = b;
}
template <bool NT>
__device__ __forceinline__ void store_state4(f16* p, const f32x4& x) {
  const u32x2v h = __builtin_bit_cast(u32x2v, __builtin_convertvector(x, f16x4));  // RNE (the default rounding mode)
  if constexpr (NT) __builtin_nontemporal_store(h, reinterpret_cast<u32x2v*>(p));
  else *reinterpret_cast<u32x2v*>(p) = h;
}

template <int DK, int DV, typename T, int GG, typename SE, bool PRO>
__global__ __launch_bounds__(512) void decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, const T* __restrict__ g,
                                                          const T* __restrict__ beta, SE* __restrict__ state,
                                                          const int* __restrict__ slots, int num_slots, int H,
                                                          T* __restrict__ o, const T* __restrict__ o_gate,
                                                          const float* __restrict__ A_log,
                                                          const float* __restrict__ dt_bias) {
  constexpr int NT = 512;
  constexpr int CG = DV / 4;         // column groups of 4 floats
  constexpr int RG = NT / CG;        // row groups
  constexpr int RPT = DK / RG;       // rows per thread
  constexpr int WAVES = NT / kWave;
  static_assert(RG * CG == NT && RPT * RG == DK, "tile does not cover the state");
  static_assert(kWave % CG == 0, "a column group must not straddle wavefronts");

  __shared__ float s_q[DK], s_k[DK], s_a[DK];
  __shared__ float s_red[WAVES][2][DV];
  __shared__ float s_qk, s_iq, s_ik;

  const int tid = threadIdx.x;
  const size_t u = blockIdx.x;  // (sequence, head) pair
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  // The state of this (sequence, head): pool slot slots[n], or n itself.
  size_t su = u;
  if (slots) {
    const int n = (int)(u / H), h = (int)(u % H);
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) {  // inactive sequence: zero output, no state access
      if (tid < DV) o[u * DV + tid] = from_f32<T>(0.f);
      return;
    }
    su = (size_t)slot * H + h;
  }
  // Issue the state loads first: they are the whole cost of the step.
  SE* S = state + su * (size_t)DK * DV;
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + RG * m;
    s[m] = load_state4(S + (size_t)r * DV + 4 * cg);
  }

  // Stage q, k and alpha = exp(g) for the key channels.
  if (tid < DK) {
    s_q[tid] = to_f32(q[u * DK + tid]);
    s_k[tid] = to_f32(k[u * DK + tid]);
    const float gx = to_f32(g[u * (DK / GG) + tid / GG]);
    float lg = kLog2e * gx;  // log2 of the decay
    if constexpr (PRO) {
      const int gi = (int)(u % H) * (DK / GG) + tid / GG;
      lg = -fast_exp2(A_log[gi] * kLog2e) * softplus_log2((gx + dt_bias[gi]) * kLog2e);
    }
    s_a[tid] = fast_exp2(lg);
  }
  __syncthreads();
  if (wave == 0) {
    float p = 0.f, sq = 0.f, sk = 0.f;
    for (int i = lane; i < DK; i += kWave) {
      p += s_q[i] * s_k[i];
      if constexpr (PRO) {
        sq += s_q[i] * s_q[i];
        sk += s_k[i] * s_k[i];
      }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      p += __shfl_xor(p, off);
      if constexpr (PRO) {
        sq += __shfl_xor(sq, off);
        sk += __shfl_xor(sk, off);
      }
    }
    if (lane == 0) {
      float iq = 1.f, ik = 1.f;
      if constexpr (PRO) {
        iq = __builtin_amdgcn_rsqf(sq + kNormEps);
        ik = __builtin_amdgcn_rsqf(sk + kNormEps);
      }
      s_iq = iq;
      s_ik = ik;
      s_qk = p * iq * ik;
    }
  }

  // Decay in registers and accumulate the two partial column reductions.
  f32x4 e = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + RG * m;
    s[m] *= s_a[r];
    e += s[m] * s_k[r];
    y += s[m] * s_q[r];
  }
  // Reduce over the row groups that share this wavefront ...
#pragma unroll
  for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      e[c] += __shfl_xor(e[c], off);
      y[c] += __shfl_xor(y[c], off);
    }
  }
  // ... then across wavefronts through LDS.
  if (lane < CG) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s_red[wave][0][4 * cg + c] = e[c];
      s_red[wave][1][4 * cg + c] = y[c];
    }
  }
  __syncthreads();
  f32x4 et = {0.f, 0.f, 0.f, 0.f}, yt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      et[c] += s_red[w][0][4 * cg + c];
      yt[c] += s_red[w][1][4 * cg + c];
    }
  }

  float b = to_f32(beta[u]);
  if constexpr (PRO) {
    b = sigmoid_f(b);
    et *= s_ik;  // reductions against the raw q, k rescaled to the unit rows
    yt *= s_iq;
  }
  const float kscale = PRO ? s_ik : 1.f;
  f32x4 vv;
#pragma unroll
  for (int c = 0; c < 4; ++c) vv[c] = to_f32(v[u * DV + 4 * cg + c]);
  const f32x4 uu = b * (vv - et);

  if (rg == 0) {
    f32x4 out = yt + s_qk * uu;
    if (o_gate) {
#pragma unroll
      for (int c = 0; c < 4; ++c) out[c] *= sigmoid_f(to_f32(o_gate[u * DV + 4 * cg + c]));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) o[u * DV + 4 * cg + c] = from_f32<T>(out[c]);
  }
  // Write-back: the workgroups of the first seven eighths of the grid stream
  // their states out with non-temporal stores; the last eighth uses ordinary
  // stores, which stay in the memory-side cache and drain under whatever runs
  // next.  The empty asm statements around the first sequence keep the
  // compiler from hoisting or sinking the two store sequences into one (which
  // drops the non-temporal hint).
  if (blockIdx.x < gridDim.x - gridDim.x / 8) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + RG * m;
      store_state4<true>(S + (size_t)r * DV + 4 * cg, s[m] + (s_k[r] * kscale) * uu);
    }
    asm volatile("" ::: "memory");
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + RG * m;
      store_state4<false>(S + (size_t)r * DV + 4 * cg, s[m] + (s_k[r] * kscale) * uu);
    }
  }
}

// Gate parameters of the prologue form (NULL A_log: the plain step).
struct Prologue {
  const float* A_log;
  const float* dt_bias;
};

template <int DK, int DV, typename T, int GG, typename SE>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                  void* state, const int* slots, int num_slots, int H, void* o, const void* o_gate,
                                  int NH, hipStream_t stream, Prologue pro) {
  if (pro.A_log)
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, T, GG, SE, true>), dim3(NH), dim3(512), 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)g, (const T*)beta, (SE*)state, slots, num_slots, H,
                       (T*)o, (const T*)o_gate, pro.A_log, pro.dt_bias);
  else
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, T, GG, SE, false>), dim3(NH), dim3(512), 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)g, (const T*)beta, (SE*)state, slots, num_slots, H,
                       (T*)o, (const T*)o_gate, nullptr, nullptr);
  return hipGetLastError();
}

template <typename T, int GG, typename SE>
static hipError_t launch_decode_g(int Dk, int Dv, const void* q, const void* k, const void* v, const void* g,
                                  const void* beta, void* state, const int* slots, int num_slots, int H, void* o,
                                  const void* o_gate, int NH, hipStream_t stream, Prologue pro) {
#define KDA_DEC(DK_, DV_)      \
  if (Dk == DK_ && Dv == DV_) \
    return launch_decode_t<DK_, DV_, T, GG, SE>(q, k, v, g, beta, state, slots, num_slots, H, o, o_gate, NH, stream, \
                                                pro);
  KDA_DEC(64, 64)
  KDA_DEC(64, 128)
  KDA_DEC(128, 64)
  KDA_DEC(128, 128)
#undef KDA_DEC
  return hipErrorInvalidValue;
}

template <typename SE>
static hipError_t launch_decode_s(bool bf16_io, int Dk, int Dv, int g_group, const void* q, const void* k,
                                  const void* v, const void* g, const void* beta, void* state, const int* slots,
                                  int num_slots, int H, void* o, const void* o_gate, int NH, hipStream_t stream,
                                  Prologue pro = {}) {
  if (bf16_io)
    return g_group == 1 ? launch_decode_g<bf16, 1, SE>(Dk, Dv, q, k, v, g, beta, state, slots, num_slots, H, o,
                                                       o_gate, NH, stream, pro)
                        : launch_decode_g<bf16, 64, SE>(Dk, Dv, q, k, v, g, beta, state, slots, num_slots, H, o,
                                                        o_gate, NH, stream, pro);
  return g_group == 1 ? launch_decode_g<float, 1, SE>(Dk, Dv, q, k, v, g, beta, state, slots, num_slots, H, o,
                                                      o_gate, NH, stream, pro)
                      : launch_decode_g<float, 64, SE>(Dk, Dv, q, k, v, g, beta, state, slots, num_slots, H, o,
                                                       o_gate, NH, stream, pro);
}

hipError_t launch_decode(bool bf16_io, int Dk, int Dv, int g_group, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* state, void* o, int NH, hipStream_t stream) {
  return launch_decode_s<float>(bf16_io, Dk, Dv, g_group, q, k, v, g, beta, state, nullptr, 0, 1, o, nullptr, NH,
                                stream);
}

hipError_t launch_decode_prologue(bool bf16_io, int Dk, int Dv, int g_group, const void* q, const void* k,
                                  const void* v, const void* g, const void* beta, float* state, void* o, int N, int H,
                                  const float* A_log, const float* dt_bias, hipStream_t stream) {
  return launch_decode_s<float>(bf16_io, Dk, Dv, g_group, q, k, v, g, beta, state, nullptr, 0, H, o, nullptr, N * H,
                                stream, Prologue{A_log, dt_bias});
}

hipError_t launch_decode_pool(bool bf16_io, int state_kind, int Dk, int Dv, int g_group, const void* q,
                              const void* k, const void* v, const void* g, const void* beta, void* pool,
                              const int* slots, int num_slots, int H, void* o, const void* o_gate, int NH,
                              const float* A_log, const float* dt_bias, hipStream_t stream) {
  const Prologue pro{A_log, dt_bias};
  if (state_kind == 1)
    return launch_decode_s<bf16>(bf16_io, Dk, Dv, g_group, q, k, v, g, beta, pool, slots, num_slots, H, o, o_gate,
                                 NH, stream, pro);
  if (state_kind == 2)
    return launch_decode_s<f16>(bf16_io, Dk, Dv, g_group, q, k, v, g, beta, pool, slots, num_slots, H, o, o_gate,
                                NH, stream, pro);
  return launch_decode_s<float>(bf16_io, Dk, Dv, g_group, q, k, v, g, beta, pool, slots, num_slots, H, o, o_gate,
                                NH, stream, pro);
}

}  // namespace kda
