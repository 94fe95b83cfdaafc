// KDA chunked prefill, gfx950 (CDNA4): one fused kernel per layer call.
//
// The chunked parallel form of the miniKimiK3 card's Kimi Delta Attention
// bullet ("Architecture" section).  The pages state that KDA trains through a
// chunked parallel form but give no algebra; the block form below is derived
// from the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t, and is exact up to rounding.  Per head and chunk of C = 64
// tokens, with S the state entering the chunk and G_r = sum_{j<=r} g_j the
// chunk-local cumulative log-decay (per key channel):
//
//   gated operands   Qt = Q*e^G, Kt = K*e^G, Kh = K*e^-G, Kb = K*e^(G_C - G)
//   k-k block        A  = strictly_lower(Diag(b) Kt Kh^T)              (MFMA)
//   q-k block        P  = lower_incl_diag(Qt Kh^T)                      (MFMA)
//   UT transform     Tm = (I + A)^-1 Diag(b): 16x16 diagonal blocks by
//                    forward substitution, off-diagonal blocks by MFMA
//   state pass       R = V - Kt S;  U = Tm R;  O = Qt S + P U;
//                    S <- Diag(e^G_C) S + Kb^T U                        (MFMA)
//
// Design for MI355X.  HBM bytes bind this path (about 100 flop per byte at
// d = 128, against a ridge near 300), so q, k, v, g, beta are read from HBM
// exactly once and o written once: the intra-chunk transform and the
// sequential state pass run in the same workgroup and hand over through LDS,
// never through HBM.  One workgroup (4 wavefronts) owns one (sequence, head,
// d_v slice) and walks that sequence's chunks in order with its fp32 state
// slice resident in MFMA accumulators.  Columns of S evolve independently, so
// splitting d_v over workgroups adds parallelism for few-head shapes; the
// slices of one head are placed on the same XCD so their shared q/k/g reads
// hit that XCD's L2.  bf16 inputs use v_mfma_f32_16x16x32_bf16 (fp32
// accumulate); float32 inputs use v_mfma_f32_16x16x4_f32 throughout.
//
// Numerics: S, A, the diagonal solve, all accumulators and e^G are fp32; MFMA
// operands (gated q/k, Tm, P, R, U and a copy of S) are rounded to the input
// type.  Decay is referenced to the chunk start, so e^-G stays finite while a
// chunk's summed log-decay per channel is above about -80.

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// MFMA helpers.  All 16x16 tiles: lane l holds D[4*(l/16) + i][l % 16].
// A is read row-major [m][k]; B is read transposed, Bt[n][k] (k contiguous).
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KSTEP = 32;
  // acc += A[16 x K] * B[K x 16]
  template <int K>
  __device__ __forceinline__ static void run(f32x4& acc, const bf16* A, int lda, const bf16* Bt, int ldb, int lane) {
    const int r = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k0 + 8 * kg);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k0 + 8 * kg);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  }
  // Runtime K (multiple of 32).
  __device__ __forceinline__ static void run_n(f32x4& acc, const bf16* A, int lda, const bf16* Bt, int ldb, int K,
                                               int lane) {
    const int r = lane & 15, kg = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 32) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k0 + 8 * kg);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k0 + 8 * kg);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  }
  // acc += A[16 x 16] * B[16 x 16], A given in float32 (converted), B transposed.
  __device__ __forceinline__ static void run16_fa(f32x4& acc, const float* A, int lda, const bf16* Bt, int ldb,
                                                  int lane) {
    const int r = lane & 15, kg = lane >> 4;
    const f32x4 af = *reinterpret_cast<const f32x4*>(A + r * lda + 4 * kg);
    bf16x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (bf16)af[i];
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(Bt + r * ldb + 4 * kg);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), acc,
                                                     0, 0, 0);
  }
  // acc += A[16 x 16] * B[16 x 16], both in bf16 (A row-major, B transposed).
  __device__ __forceinline__ static void run16(f32x4& acc, const bf16* A, int lda, const bf16* Bt, int ldb,
                                               int lane) {
    const int r = lane & 15, kg = lane >> 4;
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(A + r * lda + 4 * kg);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(Bt + r * ldb + 4 * kg);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), acc,
                                                     0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int KSTEP = 4;
  template <int K>
  __device__ __forceinline__ static void run(f32x4& acc, const float* A, int lda, const float* Bt, int ldb,
                                             int lane) {
    const int r = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + kg], Bt[r * ldb + k0 + kg], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void run_n(f32x4& acc, const float* A, int lda, const float* Bt, int ldb, int K,
                                               int lane) {
    const int r = lane & 15, kg = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + kg], Bt[r * ldb + k0 + kg], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void run16_fa(f32x4& acc, const float* A, int lda, const float* Bt, int ldb,
                                                  int lane) {
    run<16>(acc, A, lda, Bt, ldb, lane);
  }
  __device__ __forceinline__ static void run16(f32x4& acc, const float* A, int lda, const float* Bt, int ldb,
                                               int lane) {
    run<16>(acc, A, lda, Bt, ldb, lane);
  }
};

// Two adjacent elements, loaded as one 4- or 8-byte access.
__device__ __forceinline__ f32x2 load2(const bf16* p) {
  const bf16x2 x = *reinterpret_cast<const bf16x2*>(p);
  return f32x2{(float)x[0], (float)x[1]};
}
__device__ __forceinline__ f32x2 load2(const float* p) { return *reinterpret_cast<const f32x2*>(p); }
__device__ __forceinline__ void store2(bf16* p, float a, float b) {
  *reinterpret_cast<bf16x2*>(p) = bf16x2{(bf16)a, (bf16)b};
}
__device__ __forceinline__ void store2(float* p, float a, float b) { *reinterpret_cast<f32x2*>(p) = f32x2{a, b}; }
template <typename E>
__device__ __forceinline__ void store4(E* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const f32x4& v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <typename E>
__device__ __forceinline__ f32x4 load4(const E* p);
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}


template <typename T>
struct Pair;
template <>
struct Pair<bf16> {
  typedef bf16x2 type;
};
template <>
struct Pair<float> {
  typedef f32x2 type;
};
__device__ __forceinline__ f32x2 unpack2(bf16x2 x) { return f32x2{(float)x[0], (float)x[1]}; }
__device__ __forceinline__ f32x2 unpack2(f32x2 x) { return x; }

// Store N consecutive values (a contiguous run) with the widest aligned stores.
template <typename E, int N>
__device__ __forceinline__ void store_run(E* p, const float (&x)[N]) {
  if constexpr (sizeof(E) == 2) {
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 8) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (bf16)x[i + j];
        *reinterpret_cast<bf16x8*>(p + i) = v;
      }
    } else if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4)
        *reinterpret_cast<bf16x4*>(p + i) = bf16x4{(bf16)x[i], (bf16)x[i + 1], (bf16)x[i + 2], (bf16)x[i + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < N; i += 2) *reinterpret_cast<bf16x2*>(p + i) = bf16x2{(bf16)x[i], (bf16)x[i + 1]};
    }
  } else {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4)
        *reinterpret_cast<f32x4*>(p + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < N; i += 2) *reinterpret_cast<f32x2*>(p + i) = f32x2{x[i], x[i + 1]};
    }
  }
}

// ---------------------------------------------------------------------------
// Launch geometry and LDS layout.
// ---------------------------------------------------------------------------
template <int DK_, int DV_, int VS_, typename T_, int GG_>
struct PrefillCfg {
  typedef T_ T;  // input/output element type
  typedef T_ E;  // MFMA operand type (bf16 path: bf16; f32 path: float)
  static constexpr int DK = DK_, DV = DV_, VS = VS_, GG = GG_;
  static constexpr int C = 64;                   // chunk length
  static constexpr int NT = 256;                 // threads per workgroup
  static constexpr int PADE = 16 / sizeof(E);    // 16-byte row skew
  static constexpr int KP = DK + PADE;           // pitch of [*][DK] operand tiles
  static constexpr int CP = C + PADE;            // pitch of [*][C] operand tiles
  static constexpr int AP = C + 4;               // pitch of the fp32 A tile
  static constexpr int XP = 16 + PADE;           // pitch of 16x16 solve tiles
  static constexpr int PAIRS = DK / 2;           // gating: channel pairs
  static constexpr int NRB = NT / PAIRS;         // gating: row blocks
  static constexpr int RPB = C / NRB;            // gating: rows per block
  static constexpr int RT = VS / 16;             // value-column tiles per slice
  static constexpr int SMT = DK / 64;            // state row tiles per wave
  static constexpr int NS = DV / VS;             // slices per head
  static_assert(DK == 64 || DK == 128, "DK");
  static_assert(VS % 16 == 0 && DV % VS == 0, "VS");
  static_assert(NRB * PAIRS == NT && RPB * NRB == C, "gating map");
};

template <class Cfg>
struct Smem {
  typedef typename Cfg::E E;
  E q[Cfg::C][Cfg::KP];    // Qt
  E k[Cfg::C][Cfg::KP];    // Kt
  union {
    E kh[Cfg::C][Cfg::KP];  // Kh (live until A and P are formed)
    struct {
      E xt[Cfg::C][Cfg::CP];        // X^T, X = (I + A)^-1   (solve)
      E xd[4][16][Cfg::XP];         // diagonal blocks of X, row-major
      E m[4][16][Cfg::XP];          // per-wave 16x16 scratch (transposed)
    } sv;
  } u1;
  E kbt[Cfg::DK][Cfg::CP];  // Kb^T (key channel major)
  float a[Cfg::C][Cfg::AP];  // A (fp32)
  E t[Cfg::C][Cfg::CP];     // Tm row-major
  E p[Cfg::C][Cfg::CP];     // P row-major
  E vr[Cfg::VS][Cfg::CP];   // V^T, overwritten by R^T
  E uu[Cfg::VS][Cfg::CP];   // U^T
  E s[Cfg::VS][Cfg::KP];    // S^T (operand copy of the state)
  float beta[Cfg::C];
  float gam[Cfg::DK];       // e^{G_C}
  float gsum[Cfg::NRB][Cfg::DK];
};

// Lower-triangular 16x16 tiles (I, J), J <= I, in the order used for A and P.
__constant__ const int kTriI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ const int kTriJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};


template <class Cfg>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(PrefillArgs args) {
  typedef typename Cfg::T T;
  typedef typename Cfg::E E;
  constexpr int DK = Cfg::DK, DV = Cfg::DV, VS = Cfg::VS, GG = Cfg::GG, C = Cfg::C;
  constexpr int RT = Cfg::RT, SMT = Cfg::SMT, NS = Cfg::NS;
  typedef Mma<E> M;

  __shared__ Smem<Cfg> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;

  // ---- workgroup -> (unit, slice); the NS slices of a unit share an XCD ----
  const int grp = blockIdx.x / (8 * NS);
  const int w8 = blockIdx.x % (8 * NS);
  const int unit = grp * 8 + (w8 & 7);
  const int slice = w8 >> 3;
  if (unit >= args.num_units) return;
  const int H = args.H;
  const int rank = unit / H, h = unit % H;
  int seq, tok0, len;
  if (args.cu_seqlens) {
    seq = args.order ? args.order[rank] : rank;
    int a = args.cu_seqlens[seq], b = args.cu_seqlens[seq + 1];
    a = min(max(a, 0), args.T);
    b = min(max(b, a), args.T);
    tok0 = a;
    len = b - a;
  } else {
    seq = rank;
    tok0 = rank * args.T;
    len = args.T;
  }
  const int col0 = slice * VS;  // first value column of this slice

  const T* __restrict__ gq = static_cast<const T*>(args.q);
  const T* __restrict__ gk = static_cast<const T*>(args.k);
  const T* __restrict__ gv = static_cast<const T*>(args.v);
  const T* __restrict__ gg = static_cast<const T*>(args.g);
  const T* __restrict__ gb = static_cast<const T*>(args.beta);
  T* __restrict__ go = static_cast<T*>(args.o);
  const size_t state_off = ((size_t)seq * H + h) * DK * DV;

  // ---- zero the upper tiles of Tm and P once (never written afterwards) ----
  for (int idx = tid; idx < C * C; idx += Cfg::NT) {
    const int r = idx / C, c = idx % C;
    if ((c >> 4) > (r >> 4)) {
      sm.t[r][c] = from_f32<E>(0.f);
      sm.p[r][c] = from_f32<E>(0.f);
    }
  }

  // ---- initial state slice -> accumulators and operand copy ----
  // wave w owns key-channel rows [DK/4 * w, DK/4 * (w+1)), all VS columns.
  f32x4 S[SMT][RT];
#pragma unroll
  for (int mt = 0; mt < SMT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
      const int row0 = (DK / 4) * wave + 16 * mt + 4 * kg;
      const int col = 16 * nt + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][nt][i] = args.h0 ? args.h0[state_off + (size_t)(row0 + i) * DV + col0 + col] : 0.f;
      store4<E>(&sm.s[col][row0], S[mt][nt]);
    }
  }

  // ---- raw inputs of one chunk, held in registers (prefetched) ----
  // Gating map: thread = (channel pair, block of RPB consecutive tokens).
  // V map: thread = (value-column pair, block of VRPT consecutive tokens).
  constexpr int RPB = Cfg::RPB;
  constexpr int VP = VS / 2, VRG = Cfg::NT / VP, VRPT = C / VRG;
  typedef typename Pair<T>::type P2;
  const int pr = tid % Cfg::PAIRS, rb = tid / Cfg::PAIRS;
  const int ch = 2 * pr;
  const int vcp = tid % VP, vrg = tid / VP;
  P2 rq[RPB], rk[RPB], rg[GG == 1 ? RPB : 1], rv[VRPT];
  T rgs[GG == 1 ? 1 : RPB], rbeta;
  // Loads are clamped to the last valid token so that they are branch-free
  // and can all be in flight together; out-of-range rows are zeroed at use.
  auto load_raw = [&](int ck) {
    const int cbase = ck * C;
#pragma unroll
    for (int j = 0; j < RPB; ++j) {
      const int pos = min(cbase + rb * RPB + j, len - 1);
      const size_t tk = (size_t)(tok0 + pos) * H + h;
      rq[j] = *reinterpret_cast<const P2*>(gq + tk * DK + ch);
      rk[j] = *reinterpret_cast<const P2*>(gk + tk * DK + ch);
      if constexpr (GG == 1)
        rg[j] = *reinterpret_cast<const P2*>(gg + tk * DK + ch);
      else
        rgs[j] = gg[tk * (DK / GG) + ch / GG];
    }
#pragma unroll
    for (int j = 0; j < VRPT; ++j) {
      const int pos = min(cbase + vrg * VRPT + j, len - 1);
      rv[j] = *reinterpret_cast<const P2*>(gv + ((size_t)(tok0 + pos) * H + h) * DV + col0 + 2 * vcp);
    }
    if (tid < C) rbeta = gb[(size_t)(tok0 + min(cbase + tid, len - 1)) * H + h];
  };

  const int nchunks = (len + C - 1) / C;
  if (nchunks > 0) load_raw(0);
  for (int ck = 0; ck < nchunks; ++ck) {
    const int cbase = ck * C;  // token offset of the chunk within the sequence
    __syncthreads();           // previous chunk's readers are done

    // ================= phase 1: cumulative decay, gated operands ============
    {
      f32x2 qv[RPB], kv[RPB], G[RPB];
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int j = 0; j < RPB; ++j) {
        const bool ok = cbase + rb * RPB + j < len;
        f32x2 gx;
        if constexpr (GG == 1) {
          gx = unpack2(rg[j]);
        } else {
          const float gs = to_f32(rgs[j]);
          gx = f32x2{gs, gs};
        }
        const f32x2 z = {0.f, 0.f};
        qv[j] = ok ? unpack2(rq[j]) : z;
        kv[j] = ok ? unpack2(rk[j]) : z;
        gx = ok ? gx : z;
        acc0 += gx[0] * kLog2e;
        acc1 += gx[1] * kLog2e;
        G[j] = f32x2{acc0, acc1};
      }
      sm.gsum[rb][ch] = acc0;
      sm.gsum[rb][ch + 1] = acc1;
      // V slice, transposed: vr[col][token], one contiguous run per column
      {
        float v0[VRPT], v1[VRPT];
#pragma unroll
        for (int j = 0; j < VRPT; ++j) {
          const bool ok = cbase + vrg * VRPT + j < len;
          const f32x2 x = unpack2(rv[j]);
          v0[j] = ok ? x[0] : 0.f;
          v1[j] = ok ? x[1] : 0.f;
        }
        store_run<E, VRPT>(&sm.vr[2 * vcp][vrg * VRPT], v0);
        store_run<E, VRPT>(&sm.vr[2 * vcp + 1][vrg * VRPT], v1);
      }
      if (tid < C) sm.beta[tid] = cbase + tid < len ? to_f32(rbeta) : 0.f;
      __syncthreads();
      // the next chunk's raw loads fly while this chunk is computed
      if (ck + 1 < nchunks) load_raw(ck + 1);
      float off0 = 0.f, off1 = 0.f, tot0 = 0.f, tot1 = 0.f;
#pragma unroll
      for (int b = 0; b < Cfg::NRB; ++b) {
        const float x0 = sm.gsum[b][ch], x1 = sm.gsum[b][ch + 1];
        if (b < rb) {
          off0 += x0;
          off1 += x1;
        }
        tot0 += x0;
        tot1 += x1;
      }
      const float eT0 = fast_exp2(tot0), eT1 = fast_exp2(tot1);
      if (rb == 0) {
        sm.gam[ch] = eT0;
        sm.gam[ch + 1] = eT1;
      }
      float kb0[RPB], kb1[RPB];
#pragma unroll
      for (int j = 0; j < RPB; ++j) {
        const int r = rb * RPB + j;
        const float G0 = off0 + G[j][0], G1 = off1 + G[j][1];
        const float e0 = fast_exp2(G0), e1 = fast_exp2(G1);
        const float n0 = fast_exp2(-G0), n1 = fast_exp2(-G1);
        store2(&sm.q[r][ch], qv[j][0] * e0, qv[j][1] * e1);
        store2(&sm.k[r][ch], kv[j][0] * e0, kv[j][1] * e1);
        const float h0v = kv[j][0] * n0, h1v = kv[j][1] * n1;
        store2(&sm.u1.kh[r][ch], h0v, h1v);
        kb0[j] = h0v * eT0;
        kb1[j] = h1v * eT1;
      }
      store_run<E, RPB>(&sm.kbt[ch][rb * RPB], kb0);
      store_run<E, RPB>(&sm.kbt[ch + 1][rb * RPB], kb1);
    }
    __syncthreads();

    // ================= phase 2: A = strict_lower(Diag(b) Kt Kh^T), P ========
    for (int task = wave; task < 20; task += 4) {
      const int tri = task % 10;
      const int I = kTriI[tri], J = kTriJ[tri];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const E* Aop = task < 10 ? &sm.k[16 * I][0] : &sm.q[16 * I][0];
      M::template run<DK>(acc, Aop, Cfg::KP, &sm.u1.kh[16 * J][0], Cfg::KP, lane);
      const int col = 16 * J + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * I + 4 * kg + i;
        if (task < 10) {
          float val = acc[i] * sm.beta[row];
          if (col >= row) val = 0.f;
          sm.a[row][col] = val;
        } else {
          sm.p[row][col] = from_f32<E>(col > row ? 0.f : acc[i]);
        }
      }
    }
    __syncthreads();

    // ================= phase 3: Tm = (I + A)^-1 Diag(b) ====================
    if (wave == 0) {
      // Diagonal 16x16 blocks by forward substitution, fp32; lane = (block, column).
      const int blk = lane >> 4, j = lane & 15;
      const int o16 = 16 * blk;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= sm.a[o16 + r][o16 + i] * x[i];
        x[r] = s;
      }
      const float bj = sm.beta[o16 + j];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.u1.sv.xd[blk][r][j] = from_f32<E>(x[r]);
        sm.u1.sv.xt[o16 + j][o16 + r] = from_f32<E>(x[r]);
        sm.t[o16 + r][o16 + j] = from_f32<E>(x[r] * bj);
      }
    }
    __syncthreads();
    // Off-diagonal blocks, one diagonal band per level:
    //   X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      const int I = d + wave, J = wave;
      const bool act = wave < 4 - d;
      if (act) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int K = J; K < I; ++K)
          M::run16_fa(acc, &sm.a[16 * I][16 * K], Cfg::AP, &sm.u1.sv.xt[16 * J][16 * K], Cfg::CP, lane);
        store4<E>(&sm.u1.sv.m[wave][l16][4 * kg], acc);
      }
      __syncthreads();
      if (act) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        M::run16(acc, &sm.u1.sv.xd[I][0][0], Cfg::XP, &sm.u1.sv.m[wave][0][0], Cfg::XP, lane);
        acc = -acc;
        store4<E>(&sm.u1.sv.xt[16 * J + l16][16 * I + 4 * kg], acc);
        const float bj = sm.beta[16 * J + l16];
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.t[16 * I + 4 * kg + i][16 * J + l16] = from_f32<E>(acc[i] * bj);
      }
      __syncthreads();
    }

    // ================= phase 4: state pass over this slice ==================
    // 4a: R = V - Kt S and O = Qt S; wave w owns token rows [16w, 16w + 16).
    f32x4 O[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
      O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      M::template run<DK>(r, &sm.k[16 * wave][0], Cfg::KP, &sm.s[16 * nt][0], Cfg::KP, lane);
      M::template run<DK>(O[nt], &sm.q[16 * wave][0], Cfg::KP, &sm.s[16 * nt][0], Cfg::KP, lane);
      E* vp = &sm.vr[16 * nt + l16][16 * wave + 4 * kg];
      store4<E>(vp, load4<E>(vp) - r);
    }
    __syncthreads();
    // 4b: U = Tm R (Tm lower triangular: only K < 16(w+1) contributes).
    const int kmax = ((16 * (wave + 1) + M::KSTEP - 1) / M::KSTEP) * M::KSTEP;
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
      f32x4 uacc = {0.f, 0.f, 0.f, 0.f};
      M::run_n(uacc, &sm.t[16 * wave][0], Cfg::CP, &sm.vr[16 * nt][0], Cfg::CP, kmax, lane);
      store4<E>(&sm.uu[16 * nt + l16][16 * wave + 4 * kg], uacc);
    }
    __syncthreads();
    // 4c: O += P U, then write o.
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
      M::run_n(O[nt], &sm.p[16 * wave][0], Cfg::CP, &sm.uu[16 * nt][0], Cfg::CP, kmax, lane);
      const int col = col0 + 16 * nt + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = cbase + 16 * wave + 4 * kg + i;
        if (pos < len) go[((size_t)(tok0 + pos) * H + h) * DV + col] = from_f32<T>(O[nt][i]);
      }
    }
    // 4d: S <- Diag(e^{G_C}) S + Kb^T U; refresh the operand copy of S.
#pragma unroll
    for (int mt = 0; mt < SMT; ++mt) {
      const int row0 = (DK / 4) * wave + 16 * mt;
      f32x4 gm;
#pragma unroll
      for (int i = 0; i < 4; ++i) gm[i] = sm.gam[row0 + 4 * kg + i];
#pragma unroll
      for (int nt = 0; nt < RT; ++nt) {
        S[mt][nt] *= gm;
        M::template run<C>(S[mt][nt], &sm.kbt[row0][0], Cfg::CP, &sm.uu[16 * nt][0], Cfg::CP, lane);
        store4<E>(&sm.s[16 * nt + l16][row0 + 4 * kg], S[mt][nt]);
      }
    }
  }

  // ---- final state ----
  if (args.ht) {
#pragma unroll
    for (int mt = 0; mt < SMT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < RT; ++nt) {
        const int row0 = (DK / 4) * wave + 16 * mt + 4 * kg;
        const int col = 16 * nt + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) args.ht[state_off + (size_t)(row0 + i) * DV + col0 + col] = S[mt][nt][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Varlen prep: documents ordered by decreasing length (ties by index), so the
// longest chains start first.  One thread per document; O(N) scan each.
// ---------------------------------------------------------------------------
__global__ void varlen_order_kernel(const int* __restrict__ cu, int N, int T, int* __restrict__ order) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  auto length = [&](int n) {
    int a = min(max(cu[n], 0), T);
    int b = min(max(cu[n + 1], a), T);
    return b - a;
  };
  const int li = length(i);
  int r = 0;
  for (int j = 0; j < N; ++j) {
    const int lj = length(j);
    r += (lj > li) || (lj == li && j < i);
  }
  order[r] = i;
}

// Fill helpers (no hipMemsetAsync: safe to capture in graphs).
__global__ void fill_zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <class Cfg>
static hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream) {
  const int groups = (a.num_units + 7) / 8;
  const int grid = groups * 8 * Cfg::NS;
  hipLaunchKernelGGL(chunk_fwd_kernel<Cfg>, dim3(grid), dim3(Cfg::NT), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int GG>
static hipError_t launch_dims(int Dk, int Dv, int VS, const PrefillArgs& a, hipStream_t s) {
#define KDA_CASE(DK_, DV_, VS_) \
  if (Dk == DK_ && Dv == DV_ && VS == VS_) return launch_cfg<PrefillCfg<DK_, DV_, VS_, T, GG>>(a, s);
  if constexpr (sizeof(T) == 2) {
    KDA_CASE(64, 64, 64)
    KDA_CASE(64, 64, 32)
    KDA_CASE(64, 64, 16)
    KDA_CASE(64, 128, 64)
    KDA_CASE(64, 128, 32)
    KDA_CASE(128, 64, 64)
    KDA_CASE(128, 64, 32)
    KDA_CASE(128, 128, 64)
    KDA_CASE(128, 128, 32)
  } else {
    KDA_CASE(64, 64, 32)
    KDA_CASE(64, 64, 16)
    KDA_CASE(64, 128, 32)
    KDA_CASE(64, 128, 16)
  }
#undef KDA_CASE
  return hipErrorInvalidValue;
}

// Value-slice width for a shape: fill the CUs with one workgroup wave where
// possible; narrower slices cost a repeated intra-chunk transform.
int prefill_slice_width(bool bf16_io, int Dk, int Dv, long long units, int num_cus) {
  if (!bf16_io) return (Dk == 64) ? (units * (Dv / 16) <= num_cus ? 16 : 32) : 0;
  int vs = 64;
  if (Dv == 128 && units * 2 < (long long)num_cus / 2) vs = 32;
  if (Dv == 64 && units < (long long)num_cus / 2) vs = 32;
  return vs;
}

bool prefill_supported(bool bf16_io, int Dk, int Dv) { return bf16_io || Dk == 64; }

hipError_t launch_prefill(bool bf16_io, int Dk, int Dv, int g_group, int VS, const PrefillArgs& a,
                          hipStream_t stream) {
  if (bf16_io)
    return g_group == 1 ? launch_dims<bf16, 1>(Dk, Dv, VS, a, stream) : launch_dims<bf16, 64>(Dk, Dv, VS, a, stream);
  return g_group == 1 ? launch_dims<float, 1>(Dk, Dv, VS, a, stream) : launch_dims<float, 64>(Dk, Dv, VS, a, stream);
}

hipError_t launch_varlen_order(const int* cu, int N, int T, int* order, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_order_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, cu, N, T, order);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace kda
