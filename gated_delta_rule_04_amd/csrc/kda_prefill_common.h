// Device helpers shared by the KDA prefill kernels (gfx950 / CDNA4, wave64):
// MFMA operand fragments in the accumulator-matching k order, buffer-resource
// loads and stores, compile-time wavefront dispatch and the launch geometry.
#pragma once

#include "kda_common.h"

namespace kda {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// traffic, not for its global loads/stores, so prefetched global loads stay
// in flight across it (the compiler waits for them at their first use).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Compile-time wavefront roles: fn(IC<w>{}) for the uniform index w < N, so
// each wavefront's share of a stage is specialised (scalar branches only).
template <int V>
struct IC {
  static constexpr int value = V;
};
// fn(IC<0>{}), fn(IC<1>{}), ..., fn(IC<N - 1>{}), in order (compile-time indices).
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(IC<I>{});
    static_for<N, I + 1>(fn);
  }
}
template <int N, class Fn>
__device__ __forceinline__ void static_switch(int w, Fn&& fn) {
  if constexpr (N > 0) {
    if (w == N - 1)
      fn(IC<N - 1>{});
    else
      static_switch<N - 1>(w, fn);
  }
}

// A lane offset the compiler must recompute where it is used: keeps the LDS
// addresses of the per-wavefront jobs (compile-time block offsets on top)
// from being hoisted out of the chunk loop, where the variants' hoisted
// addresses together would exhaust the registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Four consecutive values to LDS: one 8-byte write (bf16) or two (fp32; fp32
// operand rows are 8-byte aligned: their pitches are skewed by 8 bytes).
template <typename E>
__device__ __forceinline__ void store4(E* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const f32x4& v) {
  *reinterpret_cast<bf16x4*>(p) = to_bf16x4(v);
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
  *reinterpret_cast<f32x2*>(p + 2) = f32x2{v[2], v[3]};
}

// N = 2 or 4 consecutive values to LDS.
template <typename E, int N>
__device__ __forceinline__ void store_run(E* p, const float (&v)[N]) {
  if constexpr (N == 4) {
    store4<E>(p, f32x4{v[0], v[1], v[2], v[3]});
  } else {
    static_assert(N == 2, "store_run");
    if constexpr (sizeof(E) == 2)
      *reinterpret_cast<unsigned*>(p) = pk_bf16(v[0], v[1]);
    else
      *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
  }
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
  else if constexpr (sizeof(P) == 8)
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  else
    return __builtin_bit_cast(P, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Eight consecutive elements, loaded with 16-byte accesses.
typedef float f32x8 __attribute__((ext_vector_type(8)));
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type load(rsrc_t r, int off) { return bload<bf16x8>(r, off); }
};
template <>
struct Vec8<float> {
  typedef f32x8 type;
  __device__ __forceinline__ static type load(rsrc_t r, int off) {
    const f32x4 a = bload<f32x4>(r, off), b = bload<f32x4>(r, off + 16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};
// CPT = 2 consecutive elements (one 4- or 8-byte access).
template <typename T, int N>
struct VecN;
template <>
struct VecN<bf16, 2> {
  typedef bf16x2 type;
  __device__ __forceinline__ static type load(rsrc_t r, int off) { return bload<bf16x2>(r, off); }
};
template <>
struct VecN<float, 2> {
  typedef f32x2 type;
  __device__ __forceinline__ static type load(rsrc_t r, int off) { return bload<f32x2>(r, off); }
};
template <typename V>
__device__ __forceinline__ float elem(const V& v, int i) {
  return (float)v[i];
}
// Sum of squares of a pair (bf16: one v_dot2_f32_bf16 on the loaded pair).
__device__ __forceinline__ float sumsq(const bf16x2& v) { return __builtin_amdgcn_fdot2_f32_bf16(v, v, 0.f, false); }
__device__ __forceinline__ float sumsq(const f32x2& v) { return v[0] * v[0] + v[1] * v[1]; }
// Four consecutive elements of a row (one 8- or 16-byte access).
template <typename T>
struct Row4;
template <>
struct Row4<bf16> {
  typedef bf16x4 type;
};
template <>
struct Row4<float> {
  typedef f32x4 type;
};
__device__ __forceinline__ void bstore4(const f32x4& v, rsrc_t r, int off, bf16) {
  const bf16x4 b = to_bf16x4(v);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), r, off, 0, 0);
}
__device__ __forceinline__ void bstore4(const f32x4& v, rsrc_t r, int off, float) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Launch geometry of the chunked prefill.  A workgroup owns one (sequence,
// head, value slice) and walks that sequence in chunks of CL tokens, each
// made of CL / 16 sub-blocks of 16 tokens.
// ---------------------------------------------------------------------------
template <int DK_, int DV_, int VS_, typename T_, int GG_, int CL_>
struct PrefillCfg {
  typedef T_ T;  // input/output element type
  typedef T_ E;  // MFMA operand type (bf16 path: bf16; f32 path: float)
  static constexpr int DK = DK_, DV = DV_, VS = VS_, GG = GG_;
  static constexpr int CL = CL_;                 // tokens per chunk (one pipeline step)
  static constexpr int NSB = CL / 16;            // 16-token sub-blocks per chunk
  static constexpr int NPW = DK / 16;            // producer wavefronts (8 or 4)
  static constexpr int NA = 64 * NPW;            // producer threads
  static constexpr int RT = VS / 16;             // value-column tiles per slice
  static constexpr int TPW = RT > 4 ? RT / 4 : 1;  // value tiles per state wavefront
  static constexpr int NBW = RT / TPW;           // state wavefronts
  static constexpr int NT = NA + 64 * NBW;       // threads per workgroup
  static constexpr int PADE = 8 / sizeof(E);     // 8-byte row skew: pitch = 2 (mod 32) dwords
  static constexpr int KP = DK + PADE;           // pitch of [*][DK] operand tiles
  // bf16: the state update's (K e^{G_end - G})^T fragments come from the
  // token-major tile through transposing LDS reads (gfx950
  // ds_read_b64_tr_b16); its rows are then 16 elements longer and
  // XOR-permuted.  fp32 reads that tile's columns directly.
  static constexpr bool TR = sizeof(E) == 2;
  static constexpr int KEP = TR ? DK + 16 : KP;  // pitch of the KE tile
  // gating: key channels per producer thread: 2, so a token row spans the
  // wavefront (128 key channels: each lane's cumulative decay is a plain
  // running sum, no cross-lane scan) or its half (64), and a lane's
  // per-channel factors serve all of its rows (8, or 4 in fp32 at 128).
  static constexpr int CPT = 2;
  static constexpr int CG = CPT < 4 ? CPT : 4;   // gating: channels per LDS write
  static constexpr int CGN = DK / CPT;           // gating: channel groups of a row
  static constexpr int NRB = NA / CGN;           // gating: row blocks
  static constexpr int RPB = CL / NRB;           // gating: rows per block
  static constexpr int RBW = 64 / CGN;           // gating: row blocks per wavefront
  static constexpr int RPW = RBW * RPB;          // gating: rows per wavefront
  static constexpr int WPB = 16 / RPW;           // gating: wavefronts per sub-block
  static constexpr int KT = DK / 16;             // key-channel tiles
  static constexpr int NS = DV / VS;             // slices per head
  static_assert(DK == 64 || DK == 128, "DK");
  static_assert(CL == 32 || CL == 64, "CL");
  static_assert(VS % 16 == 0 && DV % VS == 0 && RT % TPW == 0, "VS");
  static_assert(NRB * CGN == NA && RPB * NRB == CL && RBW * CGN == 64, "gating map");
  static_assert(RPW <= 16 && WPB * RPW == 16, "a sub-block is whole wavefronts of gating rows");
  static_assert(NSB <= NPW && NSB % 2 == 0, "one producer wavefront per sub-block transform");
  static_assert(RBW == 1 || RBW == 2, "gating: token rows of 64 or 32 lanes");
};

// Cross-lane sums without LDS traffic (the LDS is the busiest unit of the
// pipelined prefill; a __shfl_* is an LDS-crossbar ds_bpermute).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over the N = 8 or 16 consecutive lanes of a (half) row, in every lane:
// quad permutes [1,0,3,2] and [2,3,0,1], then row_half_mirror and row_mirror.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(N == 8 || N == 16, "row_sum");
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  if constexpr (N == 16) x += dpp_mov<0x140>(x);
  return x;
}
// Over the two halves of a wavefront, lane by lane: the value of the lower
// half for the upper half's lanes (0 for the lower half's) and the sum of
// both (one v_permlane32_swap).
__device__ __forceinline__ void rows2_scan(float x, int half, float& excl, float& total) {
  const unsigned xb = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  const float lower = __builtin_bit_cast(float, (unsigned)r[0]), upper = __builtin_bit_cast(float, (unsigned)r[1]);
  excl = half ? lower : 0.f;
  total = lower + upper;
}
// The total of x over the four 16-lane rows, lane by lane (the sum that
// __shfl_xor by 16 and by 32 would form).
__device__ __forceinline__ float rows4_sum(float x) {
  const unsigned xb = __builtin_bit_cast(unsigned, x);
  const auto s = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  const float pair = __builtin_bit_cast(float, (unsigned)s[0]) + __builtin_bit_cast(float, (unsigned)s[1]);
  const unsigned pb = __builtin_bit_cast(unsigned, pair);
  const auto r = __builtin_amdgcn_permlane32_swap(pb, pb, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// bf16 Kh rows: 4-element unit u of token row r is stored at unit u ^ ((r / 4) % 4).
// Row reads (16 consecutive rows), transposing reads (4 rows x 4 units per
// 16 lanes) and the producer's row writes then spread over all banks.
__device__ __forceinline__ int kh_swizzle(int row) { return (row >> 2) & 3; }


// Offset of element (r, c) of a [Dk][DV] state kept between kernels as 16x16
// tiles (tile (r/16, c/16) is 512 contiguous bytes, row-major inside): a
// wavefront's 16x16 tile is one contiguous 512-byte store, and 16 bytes of
// one row (8 columns from a multiple of 8) are one contiguous load.
template <int DV>
__device__ __forceinline__ size_t tile_off(int r, int c) {
  return (size_t)((r >> 4) * (DV / 16) + (c >> 4)) * 256 + (r & 15) * 16 + (c & 15);
}

// MFMA fragments with a k order that matches the accumulator layout, so that
// accumulators (S, R, U) feed the next product straight from registers.
// bf16 (16x16x32): slab s covers k = 32s .. 32s+31 and lane group kg holds
// k = 32s + 4kg + {0..3} and 32s + 16 + 4kg + {0..3}, i.e. rows 4kg..4kg+3 of
// accumulator tiles 2s and 2s+1.  fp32 (16x16x4): slab s covers
// k = 16(s/4) + 4kg + (s%4), i.e. element s%4 of accumulator tile s/4.
// A and B operands share this layout: lane l16 supplies row l16 of A, or
// column l16 of B, over the slab's k.  So the accumulator form of a matrix
// M (lane l: M[4(l/16) + i][l % 16]) is both M's B operand and M^T's A
// operand, and a tile loaded from row-major rows serves as an A operand of
// itself or a B operand of its transpose.
template <typename E>
struct Frag;

template <>
struct Frag<bf16> {
  typedef bf16x8 V;
  static constexpr int SLAB = 32;
  // From a row-major LDS row (the lane's row).
  __device__ __forceinline__ static V ld(const bf16* row, int s, int kg) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * s + 4 * kg);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * s + 16 + 4 * kg);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Same, from a row whose 4-element groups are XOR-permuted by sw.
  __device__ __forceinline__ static V ld_sw(const bf16* row, int s, int kg, int sw) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 4 * ((8 * s + kg) ^ sw));
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 4 * ((8 * s + 4 + kg) ^ sw));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Fragment of M^T from a token-major tile M (swizzled by kh_swizzle): the
  // lane's row of M^T is column m0 + l16 of M over slab s.  In each 16-lane
  // group a transposing read hands lane l16 element l16 % 4 of the 4-element
  // pieces addressed by lanes l16 / 4 + {0, 4, 8, 12}; so lane 4e + q of group
  // kg addresses row 32s + h + 4kg + e, elements m0 + 4q .. m0 + 4q + 3.
  template <int P>
  __device__ __forceinline__ static V ld_tr(const bf16* tile, int m0, int s, int l16, int kg) {
    const int e = l16 >> 2, q = l16 & 3;
    const bf16* lo = tile + (32 * s + 4 * kg + e) * P + 4 * ((m0 >> 2) + (q ^ kg));
    const bf16* hi = lo + 16 * P;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lo));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(hi));
    return __builtin_bit_cast(V, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  // From accumulator tiles x (tile 2s) and y (tile 2s + 1).
  __device__ __forceinline__ static V acc2(const f32x4& x, const f32x4& y) {
    return __builtin_shufflevector(to_bf16x4(x), to_bf16x4(y), 0, 1, 2, 3, 4, 5, 6, 7);
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
  __device__ __forceinline__ static V ld_sw(const float* row, int s, int kg, int sw) {
    return row[4 * ((4 * (s >> 2) + kg) ^ sw) + (s & 3)];
  }
  __device__ __forceinline__ static f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 16x16 products with both operands in accumulator form: prod(At, B) = A * B,
// where At holds A^T and B holds B.  prod(M, I) = M^T moves a tile to its
// transpose exactly (for bf16, exactly after the operand rounding).  bf16: one
// 16x16x16 MFMA on bf16-rounded operands (the transform is stored in bf16
// afterwards; the extra rounding raises its error from 1.6e-4 to 2.2e-4
// relative); fp32: four 16x16x4 steps.
template <typename E>
struct Reg16;
template <>
struct Reg16<bf16> {
  __device__ __forceinline__ static s16x4 cvt(const f32x4& x) {
    return __builtin_bit_cast(s16x4, to_bf16x4(x));
  }
  __device__ __forceinline__ static f32x4 prod(const f32x4& At, const f32x4& B) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cvt(At), cvt(B), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
  // c + the 16x16 tile given as rows (lane l16: elements 4kg..4kg+3 of row
  // l16), exact: a product with the identity, in the 16x16x32 shape of the
  // chains it joins (the rows fill k = 0..15, the upper half of k is zero).
  // An accumulator produced by one MFMA shape is never fed to another shape
  // as its C operand.
  __device__ __forceinline__ static f32x4 rows(const bf16x4& r, const f32x4& ident, const f32x4& c) {
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    const bf16x4 i4 = to_bf16x4(ident);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(r, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   __builtin_shufflevector(i4, z, 0, 1, 2, 3, 4, 5, 6, 7), c, 0, 0, 0);
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
  __device__ __forceinline__ static f32x4 rows(const f32x4& r, const f32x4& ident, const f32x4& c) {
    f32x4 d = c;
#pragma unroll
    for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_mfma_f32_16x16x4f32(r[i], ident[i], d, 0, 0, 0);
    return d;
  }
};

// (I + N)^-1 for a strictly lower 16x16 N (nilpotent, N^16 = 0), as the
// product (I + N^8)(I + N^4)(I + N^2)(I - N) = sum_{k<16} (-N)^k.
// N and Nt are N and N^T in accumulator form; returns X in accumulator form.
template <typename E>
__device__ __forceinline__ f32x4 unit_lower_inverse16(const f32x4& N, const f32x4& Nt, const f32x4& I4) {
  typedef Reg16<E> R;
  const f32x4 N2 = R::prod(Nt, N), N2t = R::prod(N, Nt);
  const f32x4 N4 = R::prod(N2t, N2), N4t = R::prod(N2, N2t);
  const f32x4 N8t = R::prod(N4, N4t);
  const f32x4 Z1 = R::prod(I4 + N2t, I4 - N);
  const f32x4 Z2 = R::prod(I4 + N4t, Z1);
  return R::prod(I4 + N8t, Z2);
}

// Operand fragment of slab s from accumulator tiles acc[0..n) along k (and
// the same for the negated tiles).
template <int N>
__device__ __forceinline__ bf16x8 acc_frag(const f32x4 (&acc)[N], int s, bf16) {
  return Frag<bf16>::acc2(acc[2 * s], acc[2 * s + 1]);
}
template <int N>
__device__ __forceinline__ float acc_frag(const f32x4 (&acc)[N], int s, float) {
  return acc[s >> 2][s & 3];
}
// Rounding to nearest even is symmetric in sign, so the negated fragment is
// the fragment with both sign bits of each packed pair flipped.
template <int N>
__device__ __forceinline__ bf16x8 acc_frag_neg(const f32x4 (&acc)[N], int s, bf16) {
  const f32x4 &x = acc[2 * s], &y = acc[2 * s + 1];
  constexpr unsigned kSign2 = 0x80008000u;
  const u32x4 p = {pk_bf16(x[0], x[1]) ^ kSign2, pk_bf16(x[2], x[3]) ^ kSign2, pk_bf16(y[0], y[1]) ^ kSign2,
                   pk_bf16(y[2], y[3]) ^ kSign2};
  return __builtin_bit_cast(bf16x8, p);
}
template <int N>
__device__ __forceinline__ float acc_frag_neg(const f32x4 (&acc)[N], int s, float) {
  return -acc[s >> 2][s & 3];
}


}  // namespace kda
