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
  // acc += A[16 x 16] * B[16 x 16] (B transposed), four 16x16x4 steps.
  template <typename TA>
  __device__ __forceinline__ static void run16_any(f32x4& acc, const TA* A, int lda, const float* Bt, int ldb,
                                                   int lane) {
    const int r = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + kg], Bt[r * ldb + k0 + kg], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void run16_fa(f32x4& acc, const float* A, int lda, const float* Bt, int ldb,
                                                  int lane) {
    run16_any(acc, A, lda, Bt, ldb, lane);
  }
  __device__ __forceinline__ static void run16(f32x4& acc, const float* A, int lda, const float* Bt, int ldb,
                                               int lane) {
    run16_any(acc, A, lda, Bt, ldb, lane);
  }
};

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// traffic, not for its global loads/stores, so prefetched global loads stay
// in flight across it (the compiler waits for them at their first use).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Completes this wave's own LDS writes before it reads them back.
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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
  *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
  *reinterpret_cast<f32x2*>(p + 2) = f32x2{v[2], v[3]};
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
  const f32x2 a = *reinterpret_cast<const f32x2*>(p), b = *reinterpret_cast<const f32x2*>(p + 2);
  return f32x4{a[0], a[1], b[0], b[1]};
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

// Store N consecutive values (a contiguous run) with 8-byte stores (LDS rows
// are 8-byte aligned: their pitches are skewed by 8 bytes against bank conflicts).
template <typename E, int N>
__device__ __forceinline__ void store_run(E* p, const float (&x)[N]) {
  if constexpr (sizeof(E) == 2) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4)
        *reinterpret_cast<bf16x4*>(p + i) = bf16x4{(bf16)x[i], (bf16)x[i + 1], (bf16)x[i + 2], (bf16)x[i + 3]};
    } else if constexpr (N % 2 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 2) *reinterpret_cast<bf16x2*>(p + i) = bf16x2{(bf16)x[i], (bf16)x[i + 1]};
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) p[i] = (bf16)x[i];
    }
  } else {
    if constexpr (N % 2 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 2) *reinterpret_cast<f32x2*>(p + i) = f32x2{x[i], x[i + 1]};
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) p[i] = x[i];
    }
  }
}

// Store NP element pairs as one contiguous run of 2*NP elements.
template <typename E, int NP>
__device__ __forceinline__ void store_pairs(E* p, const typename Pair<E>::type (&x)[NP]) {
  if constexpr (sizeof(E) == 2 && NP % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NP; i += 2)
      *reinterpret_cast<bf16x4*>(p + 2 * i) = __builtin_shufflevector(x[i], x[i + 1], 0, 1, 2, 3);
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i) *reinterpret_cast<typename Pair<E>::type*>(p + 2 * i) = x[i];
  }
}

// Raw buffer access: a per-chunk descriptor bounds every access, so loads of
// rows past the end of a sequence return zero (the inert zero padding of a
// partial chunk) and stores past the end are dropped -- no clamping, masking
// or branches.  Offsets are 32-bit byte offsets within the chunk.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename P>
__device__ __forceinline__ P bload(rsrc_t r, int off) {
  if constexpr (sizeof(P) == 2)
    return __builtin_bit_cast(P, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  else if constexpr (sizeof(P) == 4)
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  else
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Eight consecutive elements, loaded with 16-byte accesses.
typedef float f32x8 __attribute__((ext_vector_type(8)));
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type load(rsrc_t r, int off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
};
template <>
struct Vec8<float> {
  typedef f32x8 type;
  __device__ __forceinline__ static type load(rsrc_t r, int off) {
    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};
template <typename V>
__device__ __forceinline__ float elem(const V& v, int i) {
  return (float)v[i];
}

__device__ __forceinline__ void bstore(bf16 x, rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, off, 0, 0);
}
__device__ __forceinline__ void bstore(float x, rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), r, off, 0, 0);
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
  static constexpr int NPW = DK / 16;            // producer wavefronts (8 or 4)
  static constexpr int NA = 64 * NPW;            // producer threads
  static constexpr int RT = VS / 16;             // value-column tiles per slice
  static constexpr int TPW = RT > 4 ? RT / 4 : 1;  // value tiles per state wavefront
  static constexpr int NBW = RT / TPW;           // state wavefronts
  static constexpr int NT = NA + 64 * NBW;       // threads per workgroup
  static constexpr int PADE = 8 / sizeof(E);     // 8-byte row skew: pitch = 2 (mod 32) dwords
  static constexpr int KP = DK + PADE;           // pitch of [*][DK] operand tiles
  static constexpr int CP = C + PADE;            // pitch of [*][C] operand tiles
  static constexpr int AP = C + 4;               // pitch of the fp32 A tile
  static constexpr int XP = 16 + PADE;           // pitch of 16x16 solve tiles
  static constexpr int CGN = DK / 8;             // gating: groups of 8 key channels
  static constexpr int NRB = NA / CGN;           // gating: row blocks
  static constexpr int RPB = C / NRB;            // gating: rows per block
  static constexpr int RBW = 64 / CGN;           // gating: row blocks per wavefront
  static constexpr int VCG = VS / 8;             // V: groups of 8 value columns
  static constexpr int VRPT = 64 * VCG > NA ? 64 * VCG / NA : 1;  // V: rows per loading thread
  static constexpr int VTH = 64 * VCG / VRPT;    // V: loading threads
  static constexpr int KT = DK / 16;             // key-channel tiles
  static constexpr int NS = DV / VS;             // slices per head
  static_assert(DK == 64 || DK == 128, "DK");
  static_assert(VS % 16 == 0 && DV % VS == 0 && RT % TPW == 0, "VS");
  static_assert(NRB * CGN == NA && RPB * NRB == C && RPB % 2 == 0 && RBW * CGN == 64, "gating map");
  static_assert(NPW == 4 || NPW == 8, "producer wavefronts");
  static_assert(VTH <= NA && VTH * VRPT == 64 * VCG, "V map");
};

template <class Cfg>
struct Smem {
  typedef typename Cfg::E E;
  E q[Cfg::C][Cfg::KP];     // Qt = Q e^G          (token-major)
  E k[Cfg::C][Cfg::KP];     // Kt = K e^G          (token-major)
  E kh[Cfg::C][Cfg::KP];    // Kh = K e^-G         (token-major)
  E kht[Cfg::DK][Cfg::CP];  // Kh^T                (key-channel-major)
  E vt[Cfg::VS][Cfg::CP];   // V^T of the slice    (value-column-major)
  E t[Cfg::C][Cfg::CP];     // Tm = (I + A)^-1 Diag(b), row-major
  E p[Cfg::C][Cfg::CP];     // P, row-major
  alignas(16) float a[Cfg::C][Cfg::AP];  // A (fp32), rows 16-byte aligned
  alignas(16) float xd[4][16][20];  // diagonal blocks of X = (I + A)^-1, row-major (fp32)
  float beta[Cfg::C];
  alignas(16) float gam[Cfg::DK];  // e^{G_C}
  alignas(16) float gsum[Cfg::NPW][Cfg::DK];  // per-wavefront log2-decay totals
};

// MFMA fragments with a k order that matches the accumulator layout, so that
// accumulators (S, R, U) feed the next product as B operands straight from
// registers.  bf16 (16x16x32): slab s covers k = 32s .. 32s+31 and lane group
// kg holds k = 32s + 4kg + {0..3} and 32s + 16 + 4kg + {0..3}, i.e. rows
// 4kg..4kg+3 of accumulator tiles 2s and 2s+1.  fp32 (16x16x4): slab s
// covers k = 16(s/4) + 4kg + (s%4), i.e. element s%4 of accumulator tile s/4.
template <typename E>
struct Frag;

template <>
struct Frag<bf16> {
  typedef bf16x8 V;
  static constexpr int SLAB = 32;
  // From a row-major LDS row (the lane's row of an A or Bt tile).
  __device__ __forceinline__ static V ld(const bf16* row, int s, int kg) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * s + 4 * kg);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * s + 16 + 4 * kg);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // From accumulator tiles x (tile 2s) and y (tile 2s + 1).
  __device__ __forceinline__ static V acc2(const f32x4& x, const f32x4& y) {
    return V{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3], (bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
  }
  __device__ __forceinline__ static f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Frag<float> {
  typedef float V;
  static constexpr int SLAB = 4;
  __device__ __forceinline__ static V ld(const float* row, int s, int kg) {
    return row[16 * (s >> 2) + 4 * kg + (s & 3)];
  }
  __device__ __forceinline__ static f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 16x16 products with both operands in accumulator form: prod(At, B) = A * B,
// where At holds A^T and B holds B in the accumulator layout (lane l: rows
// 4(l/16) + i of column l % 16).  The accumulator form of a matrix is its
// B-operand layout and the accumulator form of its transpose is its
// A-operand layout, so chains of products never leave registers.  bf16: one
// 16x16x16 MFMA on bf16-rounded operands (the transform is stored in bf16
// afterwards; the extra rounding raises its error from 1.6e-4 to 2.2e-4
// relative); fp32: four 16x16x4 steps.
template <typename E>
struct Reg16;
template <>
struct Reg16<bf16> {
  __device__ __forceinline__ static s16x4 cvt(const f32x4& x) {
    return __builtin_bit_cast(s16x4, bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]});
  }
  __device__ __forceinline__ static f32x4 prod(const f32x4& At, const f32x4& B) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cvt(At), cvt(B), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};
template <>
struct Reg16<float> {
  __device__ __forceinline__ static f32x4 prod(const f32x4& At, const f32x4& B) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(At[i], B[i], c, 0, 0, 0);
    return c;
  }
};

// (I + N)^-1 for a strictly lower 16x16 N (nilpotent, N^16 = 0), as the
// product (I + N^8)(I + N^4)(I + N^2)(I - N) = sum_{k<16} (-N)^k.
// N and Nt are N and N^T in accumulator form; returns X in accumulator form.
template <typename E>
__device__ __forceinline__ f32x4 unit_lower_inverse16(const f32x4& N, const f32x4& Nt, int lane) {
  typedef Reg16<E> R;
  f32x4 I4;
#pragma unroll
  for (int i = 0; i < 4; ++i) I4[i] = (4 * (lane >> 4) + i == (lane & 15)) ? 1.f : 0.f;
  const f32x4 N2 = R::prod(Nt, N), N2t = R::prod(N, Nt);
  const f32x4 N4 = R::prod(N2t, N2), N4t = R::prod(N2, N2t);
  const f32x4 N8t = R::prod(N4, N4t);
  const f32x4 Z1 = R::prod(I4 + N2t, I4 - N);
  const f32x4 Z2 = R::prod(I4 + N4t, Z1);
  return R::prod(I4 + N8t, Z2);
}

// B-operand fragment of slab s from accumulator tiles acc[0..n) along k.
template <int N>
__device__ __forceinline__ bf16x8 acc_frag(const f32x4 (&acc)[N], int s, bf16) {
  return Frag<bf16>::acc2(acc[2 * s], acc[2 * s + 1]);
}
template <int N>
__device__ __forceinline__ float acc_frag(const f32x4 (&acc)[N], int s, float) {
  return acc[s >> 2][s & 3];
}

// ---------------------------------------------------------------------------
// The kernel.  Wavefronts 0-3 (producer) prepare chunk c+1 -- gating, the
// k-k and q-k blocks and the UT transform -- while wavefronts 4.. (state)
// run the state pass of chunk c.  One iteration, between LDS barriers:
//
//   X0 | producer: decay block sums, V^T, beta  | state: U = Tm R, O += P U, o
//  MID | producer: gated Qt, Kt, Kh             | state: S <- e^{G_C} (S + Kh^T U)
//   X1 | producer: A, P, diagonal solve blocks  | state: R = V - Kt S
//   X2 | producer: off-diagonal solve, Kh^T, e^G| state: O = Qt S
//
// Each state wavefront owns TPW 16-column tiles of the slice and keeps S,
// R/U and O in registers; from LDS it reads only producer outputs.
// ---------------------------------------------------------------------------
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void chunk_fwd_kernel(PrefillArgs args) {
  typedef typename Cfg::T T;
  typedef typename Cfg::E E;
  typedef Frag<E> F;
  typedef Mma<E> M;
  constexpr int DK = Cfg::DK, DV = Cfg::DV, VS = Cfg::VS, GG = Cfg::GG, C = Cfg::C;
  constexpr int NS = Cfg::NS, TPW = Cfg::TPW, KT = Cfg::KT, RPB = Cfg::RPB;
  constexpr int VP = VS / 2, VRG = Cfg::NA / VP, VRPT = C / VRG;
  constexpr int SLAB = F::SLAB;
  constexpr int SK = DK / SLAB;  // slabs over key channels
  constexpr int SC = C / SLAB;   // slabs over the chunk's tokens

  __shared__ Smem<Cfg> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int l16 = lane & 15, kg = lane >> 4;
  const bool producer = wave < Cfg::NPW;

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
  const int nchunks = (len + C - 1) / C;

  const T* __restrict__ gq = static_cast<const T*>(args.q);
  const T* __restrict__ gk = static_cast<const T*>(args.k);
  const T* __restrict__ gv = static_cast<const T*>(args.v);
  const T* __restrict__ gg = static_cast<const T*>(args.g);
  const T* __restrict__ gb = static_cast<const T*>(args.beta);
  T* __restrict__ go = static_cast<T*>(args.o);
  const size_t state_off = ((size_t)seq * H + h) * DK * DV;

  // ---- upper 16x16 tiles of Tm and P are zero and never written again ----
  for (int idx = tid; idx < C * C; idx += Cfg::NT) {
    const int r = idx / C, c = idx % C;
    if ((c >> 4) > (r >> 4)) {
      sm.t[r][c] = from_f32<E>(0.f);
      sm.p[r][c] = from_f32<E>(0.f);
    }
  }

  if (producer) {
    // ================= producer wavefronts ===================================
    // Gating map: thread = (8 key channels, block of RPB consecutive tokens);
    // the row blocks of one wavefront cover 16 consecutive tokens.
    // V map: thread = (8 value columns, VRPT consecutive tokens).
    typedef typename Vec8<T>::type V8;
    typedef typename Pair<E>::type EP2;
    constexpr int CGN = Cfg::CGN, RBW = Cfg::RBW;
    constexpr int VCG = Cfg::VCG, VRPT = Cfg::VRPT, VTH = Cfg::VTH;
    const int cg = tid % CGN, rb = tid / CGN;
    const int ch = 8 * cg;                 // first key channel of this thread
    const int rbw = lane / CGN;            // row block within the wavefront
    const int vcg = tid % VCG, vrb = tid / VCG;
    V8 rq[RPB], rk[RPB], rg[GG == 1 ? RPB : 1], rv[VRPT];
    T rgs[GG == 1 ? 1 : RPB], rbeta;
    // All loads of a chunk are in flight together; rows past the end of the
    // sequence read as zero through the per-chunk buffer bounds.
    const int rsk = H * DK * (int)sizeof(T);           // token stride of q, k (bytes)
    const int rsg = H * (DK / GG) * (int)sizeof(T);    // token stride of g
    const int rsv = H * DV * (int)sizeof(T);           // token stride of v
    const int rsb = H * (int)sizeof(T);                // token stride of beta
    // The prefetch of the next chunk is split in three parts, each issued as
    // soon as its registers are free, so that no single wave stalls on a long
    // burst of loads (the vector L1 moves about 64 bytes per clock).
    auto chunk_rows = [&](int ck) { return min(C, len - ck * C); };
    auto chunk_row0 = [&](int ck) { return (size_t)(tok0 + ck * C) * H + h; };
    auto load_gvb = [&](int ck) {  // g, v, beta
      const int nv = chunk_rows(ck);
      const size_t row0 = chunk_row0(ck);
      const rsrc_t bg = make_rsrc(gg + row0 * (DK / GG), (nv - 1) * rsg + (DK / GG) * (int)sizeof(T));
      const rsrc_t bv = make_rsrc(gv + row0 * DV + col0, (nv - 1) * rsv + VS * (int)sizeof(T));
      const rsrc_t bb = make_rsrc(gb + row0, (nv - 1) * rsb + (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) {
        const int r = rb * RPB + j;
        if constexpr (GG == 1)
          rg[j] = Vec8<T>::load(bg, r * rsg + ch * (int)sizeof(T));
        else
          rgs[j] = bload<T>(bg, r * rsg + (ch / GG) * (int)sizeof(T));
      }
      if (tid < VTH) {
#pragma unroll
        for (int j = 0; j < VRPT; ++j) rv[j] = Vec8<T>::load(bv, (vrb * VRPT + j) * rsv + 8 * vcg * (int)sizeof(T));
      }
      if (tid < C) rbeta = bload<T>(bb, tid * rsb);
    };
    auto load_q = [&](int ck) {
      const rsrc_t bq = make_rsrc(gq + chunk_row0(ck) * DK, (chunk_rows(ck) - 1) * rsk + DK * (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) rq[j] = Vec8<T>::load(bq, (rb * RPB + j) * rsk + ch * (int)sizeof(T));
    };
    auto load_k = [&](int ck) {
      const rsrc_t bk = make_rsrc(gk + chunk_row0(ck) * DK, (chunk_rows(ck) - 1) * rsk + DK * (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) rk[j] = Vec8<T>::load(bk, (rb * RPB + j) * rsk + ch * (int)sizeof(T));
    };
    float G[RPB][8];        // cumulative log2-decay of this thread's rows (block-local)
    float off[8];           // log2-decay of the chunk before this thread's block
    float eT[8];            // e^{G_C} of this thread's channels
    EP2 khp[8][RPB / 2];    // Kh of this thread's rows per channel (token pairs), for Kh^T
    f32x4 Xdiag;            // X_ww = (I + A_ww)^-1 of this wave's block, accumulator form
    // P = lower_incl_diag(Qt Kh^T) for row block IP (upper tiles stay zero)
    auto p_tiles = [&](int IP) {
      typename F::V qa[SK];
#pragma unroll
      for (int s = 0; s < SK; ++s) qa[s] = F::ld(&sm.q[16 * IP + l16][0], s, kg);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= IP) {
          typename F::V hb[SK];
#pragma unroll
          for (int s = 0; s < SK; ++s) hb[s] = F::ld(&sm.kh[16 * J + l16][0], s, kg);
          f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < SK; ++s) pacc = F::mma(qa[s], hb[s], pacc);
          const int col = 16 * J + l16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * IP + 4 * kg + i;
            float pv = pacc[i];
            if (J == IP) pv = col > row ? 0.f : pv;  // lower including the diagonal
            sm.p[row][col] = from_f32<E>(pv);
          }
        }
      }
    };
    if (nchunks > 0) {
      load_gvb(0);
      load_q(0);
      load_k(0);
    }

    for (int it = 0; it <= nchunks; ++it) {
      const int cbase = it * C;  // chunk it
      lds_barrier();  // -------------------------------------------------- X0
      if (it < nchunks) {
        // block-local cumulative decay; prefix over this wavefront's blocks
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
        for (int j = 0; j < RPB; ++j) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float gx = GG == 1 ? elem(rg[j], c) : to_f32(rgs[j]);
            acc[c] += gx * kLog2e;
            G[j][c] = acc[c];
          }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) off[c] = acc[c];  // inclusive prefix over blocks
#pragma unroll
        for (int d = 1; d < RBW; d <<= 1) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float y = __shfl_up(off[c], d * CGN);
            if (rbw >= d) off[c] += y;
          }
        }
        if (rbw == RBW - 1) {
          *reinterpret_cast<f32x4*>(&sm.gsum[wave][ch]) = f32x4{off[0], off[1], off[2], off[3]};
          *reinterpret_cast<f32x4*>(&sm.gsum[wave][ch + 4]) = f32x4{off[4], off[5], off[6], off[7]};
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) off[c] -= acc[c];  // exclusive within the wavefront
        // V^T of the slice: one contiguous run of VRPT tokens per column
        if (tid < VTH) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float vr[VRPT];
#pragma unroll
            for (int j = 0; j < VRPT; ++j) vr[j] = elem(rv[j], c);
            store_run<E, VRPT>(&sm.vt[8 * vcg + c][vrb * VRPT], vr);
          }
        }
        if (tid < C) sm.beta[tid] = to_f32(rbeta);
      }
      lds_barrier();  // ------------------------------------------------- MID
      if (it + 1 < nchunks) load_gvb(it + 1);  // prefetch (g, v, beta registers are free)
      if (it < nchunks) {
        // gated operands Qt, Kt, Kh (token-major)
        // decay before this thread's block: earlier wavefronts' totals
        for (int w = 0; w < wave; ++w) {  // uniform trip count
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.gsum[w][ch]);
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.gsum[w][ch + 4]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            off[c] += a[c];
            off[c + 4] += b[c];
          }
        }
        // the chunk's total decay: the last row block's inclusive prefix
        if (rb == Cfg::NRB - 1) {
#pragma unroll
          for (int c = 0; c < 8; ++c) eT[c] = fast_exp2(off[c] + G[RPB - 1][c]);
        }
#pragma unroll
        for (int j = 0; j < RPB; ++j) {
          const int r = rb * RPB + j;
          float e[8], n[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float Gc = off[c] + G[j][c];
            e[c] = fast_exp2(Gc);
            n[c] = fast_exp2(-Gc);
          }
          float qo[8], ko[8], ho[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float kx = elem(rk[j], c);
            qo[c] = elem(rq[j], c) * e[c];
            ko[c] = kx * e[c];
            ho[c] = kx * n[c];
            khp[c][j >> 1][j & 1] = from_f32<E>(ho[c]);
          }
          store_run<E, 8>(&sm.q[r][ch], qo);
          store_run<E, 8>(&sm.k[r][ch], ko);
          store_run<E, 8>(&sm.kh[r][ch], ho);
        }
      }
      lds_barrier();  // -------------------------------------------------- X1
      if (it + 1 < nchunks) load_q(it + 1);  // prefetch (q registers are free)
      if (it < nchunks && Cfg::NPW == 8 && wave >= 4) p_tiles(wave - 4);
      if (it < nchunks && wave < 4) {
        // A row block w (tiles J <= w, fragment loads issued up front), then
        // the diagonal block X_ww = (I + A_ww)^-1 in registers.
        const int I = wave;
        f32x4 aacc[4];
        {
          typename F::V ka[SK];
#pragma unroll
          for (int s = 0; s < SK; ++s) ka[s] = F::ld(&sm.k[16 * I + l16][0], s, kg);
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            aacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (J <= I) {
              typename F::V hb[SK];
#pragma unroll
              for (int s = 0; s < SK; ++s) hb[s] = F::ld(&sm.kh[16 * J + l16][0], s, kg);
#pragma unroll
              for (int s = 0; s < SK; ++s) aacc[J] = F::mma(ka[s], hb[s], aacc[J]);
            }
          }
        }
        // A = strictly_lower(Diag(beta) Kt Kh^T), fp32
        {
          f32x4 brow;
#pragma unroll
          for (int i = 0; i < 4; ++i) brow[i] = sm.beta[16 * I + 4 * kg + i];
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            if (J <= I) {
              const int col = 16 * J + l16;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = 16 * I + 4 * kg + i;
                aacc[J][i] *= brow[i];
                if (J == I) aacc[J][i] = col >= row ? 0.f : aacc[J][i];  // strictly lower
                sm.a[row][col] = aacc[J][i];
              }
            }
          }
        }
        lds_wave_sync();
        // diagonal block: N = A_II in accumulator form is aacc[I]; N^T from LDS
        {
          f32x4 N = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int J = 0; J < 4; ++J)
            if (J == I) N = aacc[J];
          const f32x4 Nt = *reinterpret_cast<const f32x4*>(&sm.a[16 * I + l16][16 * I + 4 * kg]);
          Xdiag = unit_lower_inverse16<E>(N, Nt, lane);
          const float bj = sm.beta[16 * I + l16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sm.xd[I][4 * kg + i][l16] = Xdiag[i];
            sm.t[16 * I + 4 * kg + i][16 * I + l16] = from_f32<E>(Xdiag[i] * bj);
          }
        }
      }
      lds_barrier();  // -------------------------------------------------- X2
      if (it + 1 < nchunks) load_k(it + 1);  // prefetch (k registers are free)
      if (it < nchunks) {
        // Off-diagonal blocks: wave J walks down block column J, which depends
        // only on its own earlier blocks (kept in registers) and on the
        // diagonal blocks:  X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ.
        if (wave < 3) {
          const int J = wave;
          const float bj = sm.beta[16 * J + l16];
          f32x4 Xc[4];  // X_KJ, K = J .. 3, accumulator form
          Xc[0] = Xdiag;
#pragma unroll
          for (int d = 1; d < 4; ++d) {
            if (J + d < 4) {
              const int I = J + d;
              f32x4 Mt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int e = 0; e < d; ++e) {
                // At = (A_{I,J+e})^T in accumulator form: lane holds A[16I + l16][16(J+e) + 4kg + i]
                const f32x4 At = *reinterpret_cast<const f32x4*>(&sm.a[16 * I + l16][16 * (J + e) + 4 * kg]);
                Mt += Reg16<E>::prod(At, Xc[e]);
              }
              const f32x4 XIt = *reinterpret_cast<const f32x4*>(&sm.xd[I][l16][4 * kg]);
              Xc[d] = -Reg16<E>::prod(XIt, Mt);
#pragma unroll
              for (int i = 0; i < 4; ++i) sm.t[16 * I + 4 * kg + i][16 * J + l16] = from_f32<E>(Xc[d][i] * bj);
            }
          }
        }
        if constexpr (Cfg::NPW == 4) p_tiles(wave);  // balances the sweeps above
        // transposed Kh and the chunk decay, read by the state pass next
#pragma unroll
        for (int c = 0; c < 8; ++c) store_pairs<E, RPB / 2>(&sm.kht[ch + c][rb * RPB], khp[c]);
        if (rb == Cfg::NRB - 1) {
          *reinterpret_cast<f32x4*>(&sm.gam[ch]) = f32x4{eT[0], eT[1], eT[2], eT[3]};
          *reinterpret_cast<f32x4*>(&sm.gam[ch + 4]) = f32x4{eT[4], eT[5], eT[6], eT[7]};
        }
      }
    }
    return;
  }

  // ================= state wavefronts ======================================
  const int bw = wave - Cfg::NPW;  // state wavefront index
  f32x4 S[TPW][KT];         // S: rows (key channels) 16mt + 4kg + i, column l16
  f32x4 R[TPW][4];          // R, then U: token rows 16t + 4kg + i
  f32x4 O[TPW][4];
  {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int col = col0 + 16 * (TPW * bw + j) + l16;
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[j][mt][i] = args.h0 ? args.h0[state_off + (size_t)(16 * mt + 4 * kg + i) * DV + col] : 0.f;
    }
  }

  const int rso = H * DV * (int)sizeof(T);  // token stride of o (bytes)
  typename F::V UF[TPW][SC];  // U as B-operand fragments (bf16 or fp32)
  for (int it = 0; it <= nchunks; ++it) {
    lds_barrier();  // -------------------------------------------------- X0
    if (it >= 1) {
      // ---- state: U = Tm R (Tm lower triangular: tile t needs k < 16(t+1)) ----
      {
        typename F::V RF[TPW][SC];
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int s = 0; s < SC; ++s) RF[j][s] = acc_frag(R[j], s, E());
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int j = 0; j < TPW; ++j) R[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          const E* trow = &sm.t[16 * t + l16][0];
#pragma unroll
          for (int s = 0; s < (16 * (t + 1) + SLAB - 1) / SLAB; ++s) {
            const typename F::V a = F::ld(trow, s, kg);
#pragma unroll
            for (int j = 0; j < TPW; ++j) R[j][t] = F::mma(a, RF[j][s], R[j][t]);
          }
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int s = 0; s < SC; ++s) UF[j][s] = acc_frag(R[j], s, E());
      }
      // ---- O += P U, then write o of chunk it - 1 ----
      const int pbase = (it - 1) * C;
      const int nv = min(C, len - pbase);
      const rsrc_t bo = make_rsrc(go + ((size_t)(tok0 + pbase) * H + h) * DV + col0, (nv - 1) * rso + VS * (int)sizeof(T));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const E* prow = &sm.p[16 * t + l16][0];
#pragma unroll
        for (int s = 0; s < (16 * (t + 1) + SLAB - 1) / SLAB; ++s) {
          const typename F::V a = F::ld(prow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j][t] = F::mma(a, UF[j][s], O[j][t]);
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          const int cb = (16 * (TPW * bw + j) + l16) * (int)sizeof(T);
#pragma unroll
          for (int i = 0; i < 4; ++i) bstore(from_f32<T>(O[j][t][i]), bo, (16 * t + 4 * kg + i) * rso + cb);
        }
      }
    }
    lds_barrier();  // ------------------------------------------------- MID
    if (it >= 1) {
      // ---- state: S <- Diag(e^{G_C}) (S + Kh^T U) ----
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        const E* krow = &sm.kht[16 * mt + l16][0];
#pragma unroll
        for (int s = 0; s < SC; ++s) {
          const typename F::V a = F::ld(krow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) S[j][mt] = F::mma(a, UF[j][s], S[j][mt]);
        }
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gam[16 * mt + 4 * kg]);
#pragma unroll
        for (int j = 0; j < TPW; ++j) S[j][mt] *= gm;
      }
    }
    lds_barrier();  // -------------------------------------------------- X1
    if (it < nchunks) {
      // ---- state: R = V - Kt S ----
      typename F::V SF[TPW][SK];  // S as B-operand fragments
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int s = 0; s < SK; ++s) SF[j][s] = acc_frag(S[j], s, E());
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) R[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const E* krow = &sm.k[16 * t + l16][0];
#pragma unroll
        for (int s = 0; s < SK; ++s) {
          const typename F::V a = F::ld(krow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) R[j][t] = F::mma(a, SF[j][s], R[j][t]);
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          const f32x4 vv = load4<E>(&sm.vt[16 * (TPW * bw + j) + l16][16 * t + 4 * kg]);
          R[j][t] = vv - R[j][t];
        }
      }
    }
    lds_barrier();  // -------------------------------------------------- X2
    if (it < nchunks) {
      // ---- state: O = Qt S ----
      typename F::V SF[TPW][SK];
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int s = 0; s < SK; ++s) SF[j][s] = acc_frag(S[j], s, E());
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) O[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const E* qrow = &sm.q[16 * t + l16][0];
#pragma unroll
        for (int s = 0; s < SK; ++s) {
          const typename F::V a = F::ld(qrow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j][t] = F::mma(a, SF[j][s], O[j][t]);
        }
      }
    }
  }

  // ---- final state ----
  if (args.ht) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int col = col0 + 16 * (TPW * bw + j) + l16;
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) args.ht[state_off + (size_t)(16 * mt + 4 * kg + i) * DV + col] = S[j][mt][i];
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
    KDA_CASE(64, 128, 128)
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
  // widest slice that still gives every CU a workgroup (64 at most with 128
  // key channels: wider state slices do not fit the register budget)
  for (int vs = (Dk == 128 ? 64 : Dv); vs > 32; vs /= 2)
    if (units * (Dv / vs) >= num_cus / 2) return vs;
  return 32;
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
