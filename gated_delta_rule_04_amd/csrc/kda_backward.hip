// KDA backward pass of the chunked form, gfx950 (CDNA4), bf16 inputs.
//
// The miniKimiK3 card ("Architecture", Kimi Delta Attention bullet) states
// that KDA trains through a chunked parallel form; training needs the
// gradients of a loss L = <do, o> + <dht, ht> with respect to q, k, v, g,
// beta and h0.  The block algebra below is the reverse mode of the chunked
// forward (same notation: per head and chunk, G the chunk-local cumulative
// log-decay, Qt = Q e^G, Kt = K e^G, Kh = K e^-G, gam = e^{G_last},
// A = strictly_lower(Diag(b) Kt Kh^T), P = lower_incl(Qt Kh^T),
// X = (I + A)^-1, T = X Diag(b)):
//
// 1. The forward keeps the state S entering every chunk (bf16, as 16x16
//    tiles: tile_off).
// 2. chunk_bwd_prep_kernel, per chunk, independently: with W = T Kt and
//    Z = Qt - P W, the state cotangent crosses the chunk as
//        dS_in = F^T dS_out + b,  F = Diag(gam)(I - Kh^T W),  b = Z^T dO
//    (F is the chunk's forward map S -> Diag(gam) S + Kb^T U on S).
// 3. chunk_bwd_dh_kernel walks each sequence's chunks backwards from dht,
//    keeping dS_out of every chunk (bf16), and returns dh0 (fp32).
// 4. chunk_bwd_local_kernel, per chunk, independently, with S and
//    dSt = Diag(gam) dS_out:
//        R = V - Kt S;  U = T R;  dU = Kh dSt + P^T dO;  dR = T^T dU (= dv)
//        dP = lower_incl(dO U^T);  dT = lower_incl(dU R^T)
//        dbeta_j = sum_i dT_ij X_ij + sum_i dA_ji B_ji  (B = Kt Kh^T)
//        dA = -strict(X^T dT Diag(b) X^T);  dB = Diag(b) dA
//        dQt = dO S^T + dP Kh;  dKt = -dR S^T + dB Kh
//        dKh' = dB^T Kt + dP^T Qt;  dKb = U dSt^T
//        dq = dQt e^G;  dk = dKt e^G + (dKh' + dKb) e^-G
//        dG = q dq + k (dKt e^G - (dKh' + dKb) e^-G), plus on the chunk's
//             last row sum_r (dKb * Kh)_r + rowsum(S * dSt);
//        dg = reverse cumulative sum of dG over the chunk (summed over a
//             decay group when one log-decay value serves 64 channels).
//
// Decay references.  Written with chunk-start factors, Kh = K e^{-G} grows as
// e^{-G} and leaves fp32 once a channel's decay over the chunk passes about
// -88.  No factor here is referenced further away than one 16-token block:
// the operand rows are stored as qt = Q e^{G - m}, kt = K e^{G - m},
// kh = K e^{m - G} with m the midpoint of the row's block (factors within
// e^{|block sum| / 2}); a product of block-I rows with block-J rows (I > J)
// carries the per-channel shift e^{m_I - m_J} <= 1 on one operand; the state
// side uses Kt = kt e^{m}, Qt = qt e^{m} and Kb = Kh Diag(gam) = kh e^{G_last - m}
// (all <= 1).  Every product equals its chunk-start form exactly (the
// references cancel), so the gradients are taken with the references held
// constant, and the path is exact while every 16-token block's decay sum
// stays above about -170 per channel.
//
// Design for MI355X.  Steps 2 and 4 are fully parallel over (chunk, head):
// one workgroup per chunk-head, one wavefront per 16 key channels, all
// operand tiles in LDS and every product on v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation.  LDS tiles are stored with their 4-element units
// XOR-permuted by row / 4, so one copy serves both row reads and transposing
// reads (ds_read_b64_tr_b16).  Step 4 walks the value columns in slices of 32
// to stay inside the 160 KB of LDS per workgroup; everything that contracts
// over the value axis accumulates in registers across the slices; the next
// slice's global loads are in flight while the current one is computed.
// Step 3 is the only recurrence: a short MFMA chain per chunk, with F^T and
// b (bf16) fetched two chunks ahead.  The slot of chunk c of the sequence
// that starts at token t0 and has index n is (t0 / 64) + n + c, so the
// per-chunk buffers need no prefix sum over the sequences.

#include "kda_prefill_common.h"
#include "kda_launch.h"

#ifndef KDA_BWD_DH_WAVES
#define KDA_BWD_DH_WAVES 4  // wavefronts (16-column tiles) per reverse-state-pass workgroup
#endif
#ifndef KDA_BWD_DH_STAGES
#define KDA_BWD_DH_STAGES 2  // chunks of F^T and b in flight ahead of the reverse state pass
#endif

namespace kda {

namespace {

template <int DK_, int DV_, int GG_>
struct BwdCfg {
  static constexpr int DK = DK_, DV = DV_, GG = GG_;
  static constexpr int C = 64;
  static constexpr int NW = DK / 16;   // wavefronts: one per 16 key channels
  static constexpr int NT = 64 * NW;
  static constexpr int NB = NT / DK;   // gating: token blocks per chunk
  static constexpr int TB = C / NB;    // gating: tokens per block
  static constexpr int KHP = DK + 16;  // pitch of the [C][DK] operand tiles
  static constexpr int CTP = C + 16;   // pitch of the [C][C] tiles
  static constexpr int AP = C + 4;     // pitch of the fp32 A tile
  static constexpr int VSL = 32;       // local kernel: value columns per slice
  static constexpr int SP = VSL + 16;  // pitch of the slice tiles
  static constexpr int DVP = DV + 16;  // pitch of the [C][DV] dO tile (prep)
  static_assert(NB == 4 && TB == 16, "gating map");
};

typedef Frag<bf16> F;
typedef F::V FV;

// Element offset of column c within row r of a unit-swizzled tile.
__device__ __forceinline__ int swz(int r, int c) { return 4 * ((c >> 2) ^ kh_swizzle(r)) + (c & 3); }

// Row fragment (slab s) of row `row` of a unit-swizzled tile with pitch P.
template <int P>
__device__ __forceinline__ FV ld_row(const bf16* tile, int row, int s, int kg) {
  return F::ld_sw(tile + row * P, s, kg, kh_swizzle(row));
}

// Four consecutive values of row r, columns c .. c+3 (c % 4 == 0) of a swizzled tile.
template <int P>
__device__ __forceinline__ void st_row4(bf16* tile, int r, int c, const f32x4& v) {
  store4<bf16>(tile + r * P + swz(r, c), v);
}

// An accumulator tile M (lane: M[4kg+i][l16]) at block (R0, C0) of a swizzled
// tile, written as rows through the exact transposing product.
template <int P>
__device__ __forceinline__ void st_acc(bf16* tile, int R0, int C0, const f32x4& m, const f32x4& ident, int l16,
                                       int kg) {
  st_row4<P>(tile, R0 + l16, C0 + 4 * kg, Reg16<bf16>::prod(m, ident));
}
// The same tile written transposed: tile[C0 + j][R0 + i] = M[i][j].
template <int P>
__device__ __forceinline__ void st_acc_t(bf16* tile, int R0, int C0, const f32x4& m, int l16, int kg) {
  st_row4<P>(tile, C0 + l16, R0 + 4 * kg, m);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The lower 16x16 tiles (I >= J) of a 64x64 matrix, the diagonal ones first.
__device__ __forceinline__ void lower_tile(int j, int& I, int& J) {
  // 0..3: (0,0) (1,1) (2,2) (3,3); 4..9: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
  if (j < 4) {
    I = J = j;
  } else {
    const int o = j - 4;
    I = o < 1 ? 1 : (o < 3 ? 2 : 3);
    J = o - (I == 1 ? 0 : (I == 2 ? 1 : 3));
  }
}

// A bf16 operand fragment scaled elementwise: elements 0..3 by lo, 4..7 by hi
// (rounded to nearest even).
__device__ __forceinline__ FV scale8(const FV& a, const f32x4& lo, const f32x4& hi) {
  const f32x4 x = f32x4{(float)a[0], (float)a[1], (float)a[2], (float)a[3]} * lo;
  const f32x4 y = f32x4{(float)a[4], (float)a[5], (float)a[6], (float)a[7]} * hi;
  return __builtin_shufflevector(to_bf16x4(x), to_bf16x4(y), 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 splat4(float x) { return f32x4{x, x, x, x}; }
// The per-channel values of v for the 8 channels of a row fragment of slab s
// (channels 32s + 4kg .. +3 and 32s + 16 + 4kg .. +3).
__device__ __forceinline__ void row_vals(const float* v, int s, int kg, f32x4& lo, f32x4& hi) {
  lo = *reinterpret_cast<const f32x4*>(v + 32 * s + 4 * kg);
  hi = *reinterpret_cast<const f32x4*>(v + 32 * s + 16 + 4 * kg);
}
// e^{a_c - b_c} (a, b in log2 units) for the channels of a row fragment of slab s.
__device__ __forceinline__ void row_shift(const float* a, const float* b, int s, int kg, f32x4& lo, f32x4& hi) {
  f32x4 a0, a1, b0, b1;
  row_vals(a, s, kg, a0, a1);
  row_vals(b, s, kg, b0, b1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = fast_exp2(a0[i] - b0[i]);
    hi[i] = fast_exp2(a1[i] - b1[i]);
  }
}

// Sequence geometry shared by the kernels.
struct Seq {
  int seq, tok0, len;
};
__device__ __forceinline__ Seq seq_info(const int* cu, int n, int T) {
  Seq s;
  s.seq = n;
  if (cu) {
    const int a = min(max(cu[n], 0), T);
    const int b = min(max(cu[n + 1], a), T);
    s.tok0 = a;
    s.len = b - a;
  } else {
    s.tok0 = n * T;
    s.len = T;
  }
  return s;
}
// The sequence and chunk of a slot: the last n with base(n) = t0(n) / 64 + n
// <= slot (base is strictly increasing); the slot is unused if its chunk
// index is past the sequence's chunks.
__device__ __forceinline__ bool slot_chunk(const int* cu, int N, int T, int slot, Seq& s, int& c) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const Seq m = seq_info(cu, mid, T);
    if ((m.tok0 >> 6) + mid <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  s = seq_info(cu, lo, T);
  c = slot - ((s.tok0 >> 6) + lo);
  return c >= 0 && c * 64 < s.len;
}

}  // namespace


// ---------------------------------------------------------------------------
// The chunk front of the parallel kernels: gating, the k-k and q-k blocks and
// the UT solve, all into LDS.  The prep kernel (LOCAL false) forms T and P
// rows and stores the X, T and P^T blocks to the workspace; the local kernel
// (LOCAL true) gates its chunk the same way and builds its tiles (T, T^T, P^T,
// X rows) from those blocks instead of forming them again.
// ---------------------------------------------------------------------------
template <class Cfg>
struct FrontTiles {
  static constexpr int C = Cfg::C, KHP = Cfg::KHP, CTP = Cfg::CTP, DK = Cfg::DK;
  bf16 qt[C * KHP], kt[C * KHP], kh[C * KHP];  // swizzled token-major
  bf16 t[C * CTP];   // T rows
  bf16 u1[C * CTP];  // local: T^T rows; prep: P rows
  bf16 u2[C * CTP];  // local: P^T rows
  bf16 x[C * CTP];   // local: X rows
  alignas(16) float gam[DK];    // e^{G_last}
  alignas(16) float glast[DK];  // G_last (log2 units)
  alignas(16) float beta[C];
  // the blocks' decay sums while gating; afterwards the block references m_b
  // (log2 units, the midpoint of block b's decay, chunk-relative)
  alignas(16) float gsum[Cfg::NB][DK];
  alignas(16) float em[Cfg::NB][DK];  // e^{m_b}: block-referenced rows -> chunk start
  alignas(16) float eb[Cfg::NB][DK];  // e^{G_last - m_b}: block-referenced rows -> chunk end
};
template <class Cfg>
struct FrontScratch {
  alignas(16) float a[Cfg::C * Cfg::AP];  // A = Diag(b) B below the diagonal blocks (fp32)
  alignas(16) float xd[4][16][20];        // diagonal blocks of X (fp32)
};

template <class Cfg, bool LOCAL>
__device__ __forceinline__ void chunk_front(const BwdArgs& A, const Seq& sq, int h, int c, FrontTiles<Cfg>& ft,
                                            FrontScratch<Cfg>& fs, float (&G2)[Cfg::TB], float& offref, float& mref,
                                            float& glref, const f32x4& ident) {
  constexpr int DK = Cfg::DK, C = Cfg::C, GG = Cfg::GG, KHP = Cfg::KHP, CTP = Cfg::CTP, AP = Cfg::AP;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, TB = Cfg::TB, SK = DK / 32;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = A.H;

  // The front's lower 16x16 blocks of X (set 0), T (set 1) and P^T (set 2),
  // block b in lower_tile order, in accumulator lane order: the prep kernel
  // stores the ones it forms, the local kernel reads them instead of forming
  // them again (the same values, rounded to bf16 where both kernels round).
  bf16* const tw = A.tw + ((size_t)((sq.tok0 >> 6) + sq.seq + c) * H + h) * (kFrontTileBytes / 2);
  auto tile_at = [&](int set, int b) { return tw + ((size_t)(set * 10 + b) * 64 + lane) * 4; };
  constexpr int NJB = (10 + NW - 1) / NW;  // blocks per wave
  bf16x4 tl[NJB][3];
  if constexpr (LOCAL) {  // issued first: they land while the gating runs
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      const int j = min(wave + NW * jb, 9);
#pragma unroll
      for (int set = 0; set < 3; ++set) tl[jb][set] = *reinterpret_cast<const bf16x4*>(tile_at(set, j));
    }
  }

  // ---- zero the C x C tiles (their zero parts are never written) ----
  {
    bf16* base = ft.t;
    constexpr int n = 4 * C * CTP / 4;  // 8-byte units of t, u1, u2, x (contiguous)
    static_assert(sizeof(bf16) * C * CTP * 4 == 8 * n, "tile block");
    for (int i = tid; i < n; i += NT) *reinterpret_cast<u32x2*>(base + 4 * i) = u32x2{0u, 0u};
  }

  // ---- gating: thread = (key channel, block of 16 tokens) ----
  const int nv = min(C, sq.len - c * C);
  const size_t row0 = (size_t)(sq.tok0 + c * C) * H + h;
  const int rsk = H * DK * 2, rsg = H * (DK / GG) * 2, rsb = H * 2;
  const rsrc_t bq = make_rsrc(A.q + row0 * DK, (nv - 1) * rsk + DK * 2);
  const rsrc_t bk = make_rsrc(A.k + row0 * DK, (nv - 1) * rsk + DK * 2);
  const rsrc_t bg = make_rsrc(A.g + row0 * (DK / GG), (nv - 1) * rsg + (DK / GG) * 2);
  const int ch = tid % DK, tb = tid / DK;
  bf16 qv[TB], kv[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int r = tb * TB + j;
    qv[j] = bload<bf16>(bq, r * rsk + ch * 2);
    kv[j] = bload<bf16>(bk, r * rsk + ch * 2);
  }
  {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int r = tb * TB + j;
      acc += to_f32(bload<bf16>(bg, r * rsg + (ch / GG) * 2)) * kLog2e;
      G2[j] = acc;
    }
    ft.gsum[tb][ch] = acc;
    if (tid < C) {
      const rsrc_t bb = make_rsrc(A.beta + row0, (nv - 1) * rsb + 2);
      ft.beta[tid] = to_f32(bload<bf16>(bb, tid * rsb));
    }
  }
  __syncthreads();
  {
    float off = 0.f;
    for (int b = 0; b < tb; ++b) off += ft.gsum[b][ch];
    // the block's reference: the midpoint of its decay, so that the factors
    // e^{+-(G - m)} of its rows stay within e^{|block sum| / 2}
    const float m = off + 0.5f * ft.gsum[tb][ch];
    mref = m;
    offref = off;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      G2[j] += off;
      const int r = tb * TB + j;
      const float q = to_f32(qv[j]), kk = to_f32(kv[j]);
      const float eu = fast_exp2(G2[j] - m), ed = fast_exp2(m - G2[j]);
      const int o = r * KHP + swz(r, ch);
      ft.qt[o] = (bf16)(q * eu);
      ft.kt[o] = (bf16)(kk * eu);
      ft.kh[o] = (bf16)(kk * ed);
    }
    if (tb == Cfg::NB - 1) {
      ft.gam[ch] = fast_exp2(G2[TB - 1]);
      ft.glast[ch] = G2[TB - 1];
    }
    __syncthreads();  // every thread has read the block sums
    ft.gsum[tb][ch] = m;
    ft.em[tb][ch] = fast_exp2(m);
  }
  __syncthreads();
  glref = ft.glast[ch];
  ft.eb[tb][ch] = fast_exp2(glref - mref);

  auto rows = [&](FV (&fr)[SK], const bf16* tile, int blk) {
#pragma unroll
    for (int s = 0; s < SK; ++s) fr[s] = ld_row<KHP>(tile, 16 * blk + l16, s, kg);
  };
  auto mma_rows = [&](const FV (&a)[SK], const FV (&b)[SK]) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < SK; ++s) acc = F::mma(a[s], b[s], acc);
    return acc;
  };

  if constexpr (LOCAL) {
    // T rows, T^T rows, X rows and P^T rows from the prep kernel's blocks
    auto f32 = [](const bf16x4& b) { return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]}; };
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      const int j = wave + NW * jb;
      if (j < 10) {
        int I, J;
        lower_tile(j, I, J);
        const f32x4 X = f32(tl[jb][0]), Tb = f32(tl[jb][1]), Pr = f32(tl[jb][2]);
        st_acc<CTP>(ft.t, 16 * I, 16 * J, Tb, ident, l16, kg);
        st_acc_t<CTP>(ft.u1, 16 * I, 16 * J, Tb, l16, kg);
        st_acc<CTP>(ft.x, 16 * I, 16 * J, X, ident, l16, kg);
        st_acc<CTP>(ft.u2, 16 * J, 16 * I, Pr, ident, l16, kg);  // Pr: P_IJ^T in accumulator form
      }
    }
    __syncthreads();
    return;
  }

  // ---- diagonal blocks (waves 0..3) and the blocks below them ----
  f32x4 Xdiag = zero4();
  for (int j = wave; j < 10; j += NW) {
    int I, J;
    lower_tile(j, I, J);
    if (j < 4) {
      FV ktr[SK], khr[SK], qtr[SK];
      rows(ktr, ft.kt, I);
      rows(khr, ft.kh, I);
      rows(qtr, ft.qt, I);
      f32x4 N = mma_rows(ktr, khr), Nt = mma_rows(khr, ktr);
      const float bl = ft.beta[16 * I + l16];
      const f32x4 br = *reinterpret_cast<const f32x4*>(&ft.beta[16 * I + 4 * kg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * kg + i;
        N[i] = l16 < r ? N[i] * br[i] : 0.f;
        Nt[i] = r < l16 ? Nt[i] * bl : 0.f;
      }
      // P rows: lane holds P[l16][4kg+i] (P_II^T in accumulator form)
      f32x4 Pt = mma_rows(khr, qtr);
#pragma unroll
      for (int i = 0; i < 4; ++i) Pt[i] = 4 * kg + i <= l16 ? Pt[i] : 0.f;
      st_row4<CTP>(ft.u1, 16 * I + l16, 16 * I + 4 * kg, Pt);
      Xdiag = unit_lower_inverse16<bf16>(N, Nt, ident);
      *reinterpret_cast<f32x4*>(&fs.xd[I][l16][4 * kg]) = Reg16<bf16>::prod(Xdiag, ident);
      const f32x4 Td = Xdiag * bl;  // T_II = X_II Diag(b), columns scaled
      st_acc<CTP>(ft.t, 16 * I, 16 * I, Td, ident, l16, kg);
      *reinterpret_cast<bf16x4*>(tile_at(0, j)) = to_bf16x4(Xdiag);  // for the local kernel
      *reinterpret_cast<bf16x4*>(tile_at(1, j)) = to_bf16x4(Td);
      *reinterpret_cast<bf16x4*>(tile_at(2, j)) = to_bf16x4(Pt);
    } else {
      FV ktr[SK], khr[SK], qtr[SK];
      rows(ktr, ft.kt, I);
      rows(khr, ft.kh, J);
      rows(qtr, ft.qt, I);
      // the pair's reference shift e^{m_I - m_J} (<= 1) on the block-I operands
#pragma unroll
      for (int s = 0; s < SK; ++s) {
        f32x4 lo, hi;
        row_shift(ft.gsum[I], ft.gsum[J], s, kg, lo, hi);
        ktr[s] = scale8(ktr[s], lo, hi);
        qtr[s] = scale8(qtr[s], lo, hi);
      }
      // A_IJ rows: lane holds B[16I + l16][16J + 4kg + i], scaled by b of its row
      const f32x4 Bt = mma_rows(khr, ktr) * ft.beta[16 * I + l16];
      *reinterpret_cast<f32x4*>(&fs.a[(16 * I + l16) * AP + 16 * J + 4 * kg]) = Bt;
      const f32x4 Pt = mma_rows(khr, qtr);  // P rows (P_IJ^T in accumulator form)
      st_row4<CTP>(ft.u1, 16 * I + l16, 16 * J + 4 * kg, Pt);
      *reinterpret_cast<bf16x4*>(tile_at(2, j)) = to_bf16x4(Pt);
    }
  }
  __syncthreads();

  // ---- blocks of X below the diagonal, column J on wave J:
  //      X_IJ = -X_II sum_{K=J}^{I-1} A_IK X_KJ ----
  static_switch<3>(wave, [&](auto Jc) {
    constexpr int J = decltype(Jc)::value;
    const float bj = ft.beta[16 * J + l16];
    f32x4 Xc[4 - J];
    Xc[0] = Xdiag;
#pragma unroll
    for (int d = 1; d < 4 - J; ++d) {
      const int I = J + d;
      f32x4 M = zero4();
#pragma unroll
      for (int e = 0; e < d; ++e) {
        const f32x4 At = *reinterpret_cast<const f32x4*>(&fs.a[(16 * I + l16) * AP + 16 * (J + e) + 4 * kg]);
        M += Reg16<bf16>::prod(At, Xc[e]);
      }
      const f32x4 XIt = *reinterpret_cast<const f32x4*>(&fs.xd[I][l16][4 * kg]);
      Xc[d] = -Reg16<bf16>::prod(XIt, M);
      const f32x4 Tn = Xc[d] * bj;
      st_acc<CTP>(ft.t, 16 * I, 16 * J, Tn, ident, l16, kg);
      const int b = 4 + I * (I - 1) / 2 + J;  // lower_tile's index of block (I, J)
      *reinterpret_cast<bf16x4*>(tile_at(0, b)) = to_bf16x4(Xc[d]);  // for the local kernel
      *reinterpret_cast<bf16x4*>(tile_at(1, b)) = to_bf16x4(Tn);
    }
  });
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Step 2: per chunk-head, the transfer F^T and the offset b of the state
// cotangent.  Wave w owns key-channel tile w: W and Z columns, F column tile
// w (its F^T row tile), and b row tile w.
// ---------------------------------------------------------------------------
template <class Cfg>
struct PrepSmem {
  FrontTiles<Cfg> ft;
  union {
    FrontScratch<Cfg> fs;
    bf16 dO[Cfg::C * Cfg::DVP];
  } u;
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void chunk_bwd_prep_kernel(BwdArgs A) {
  constexpr int DK = Cfg::DK, DV = Cfg::DV, C = Cfg::C, KHP = Cfg::KHP, CTP = Cfg::CTP, DVP = Cfg::DVP;
  constexpr int NT = Cfg::NT, KS = DK / 32;
  __shared__ PrepSmem<Cfg> sm;
  const int h = blockIdx.x % A.H, slot = blockIdx.x / A.H;
  Seq sq;
  int c;
  if (!slot_chunk(A.cu_seqlens, A.N, A.T, slot, sq, c)) return;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x4 ident;
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (4 * kg + i == l16) ? 1.f : 0.f;
  // dO of the chunk, 16-byte pieces, fetched before the front and stored to
  // LDS (swizzled token-major) after it
  constexpr int NP = C * DV / 8 / NT;
  static_assert(NP * NT * 8 == C * DV, "dO pieces");
  const int nv = min(C, sq.len - c * C);
  const size_t row0 = (size_t)(sq.tok0 + c * C) * A.H + h;
  const int rsv = A.H * DV * 2;
  u32x4 op[NP];
  {
    const rsrc_t bo = make_rsrc(A.dout + row0 * DV, (nv - 1) * rsv + DV * 2);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = tid + NT * j, r = p / (DV / 8), c8 = 8 * (p % (DV / 8));
      op[j] = bload<u32x4>(bo, r * rsv + c8 * 2);
    }
  }
  float G2[Cfg::TB], offref, mref, glref;
  chunk_front<Cfg, false>(A, sq, h, c, sm.ft, sm.u.fs, G2, offref, mref, glref, ident);
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int p = tid + NT * j, r = p / (DV / 8), c8 = 8 * (p % (DV / 8));
    *reinterpret_cast<u32x2*>(&sm.u.dO[r * DVP + swz(r, c8)]) = u32x2{op[j][0], op[j][1]};
    *reinterpret_cast<u32x2*>(&sm.u.dO[r * DVP + swz(r, c8 + 4)]) = u32x2{op[j][2], op[j][3]};
  }

  // W = T Kt (column tile w, all token tiles), Z = Qt - P W, with the
  // chunk-start forms Kt = kt e^{m}, Qt = qt e^{m} of the block-referenced
  // tiles (factors <= 1; lane channel 16w + l16)
  const int cw = 16 * w + l16;
  f32x4 W[4], Z[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (32 * s <= 16 * tt + 15)
        acc = F::mma(ld_row<CTP>(sm.ft.t, 16 * tt + l16, s, kg),
                     scale8(F::ld_tr<KHP>(sm.ft.kt, 16 * w, s, l16, kg), splat4(sm.ft.em[2 * s][cw]),
                            splat4(sm.ft.em[2 * s + 1][cw])),
                     acc);
    W[tt] = acc;
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    f32x4 pw = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (32 * s <= 16 * tt + 15)
        pw = F::mma(ld_row<CTP>(sm.ft.u1, 16 * tt + l16, s, kg), F::acc2(W[2 * s], W[2 * s + 1]), pw);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * tt + 4 * kg + i;
      Z[tt][i] = (float)sm.ft.qt[r * KHP + swz(r, cw)] * sm.ft.em[tt][cw] - pw[i];
    }
  }
  __syncthreads();  // dO complete

  const size_t uh = (size_t)slot * A.H + h;
  // F = Diag(gam)(I - Kh^T W) = Diag(gam) - M, M = Kb^T W with Kb = Kh
  // Diag(gam) = kh e^{G_last - m} (factors <= 1).  The decay part is kept
  // apart (gam, fp32) and applied exactly by the reverse pass; only -M, a
  // correction that is small where the chain is long and undamped, is rounded
  // to bf16.  Rounding F whole would round its near-1 diagonal in every chunk.
  // Tile (r, w) of -M is stored as A-operand fragments of -M^T,
  // [row tile w][slab][lane][8]: elements 0..3 from tile r = 2s, 4..7 from r = 2s + 1.
  if (tid < DK) A.gw[uh * DK + tid] = sm.ft.gam[tid];
  // (the two tiles of a fragment are stored together: one contiguous
  // 16-byte piece per lane, 1 KB per wavefront store)
  bf16* fw = A.fw + uh * DK * DK;
#pragma unroll
  for (int r2 = 0; r2 < DK / 32; ++r2) {
    bf16x4 half[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * r2 + e;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int cr = 16 * r + l16;
        const FV kb = scale8(F::ld_tr<KHP>(sm.ft.kh, 16 * r, s, l16, kg), splat4(sm.ft.eb[2 * s][cr]),
                             splat4(sm.ft.eb[2 * s + 1][cr]));
        acc = F::mma(kb, F::acc2(W[2 * s], W[2 * s + 1]), acc);
      }
      half[e] = to_bf16x4(-acc);
    }
    *reinterpret_cast<FV*>(fw + ((size_t)(w * KS + r2) * 64 + lane) * 8) =
        __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // b = Z^T dO, bf16 accumulator tiles [row tile w][column tile][lane][4]
  bf16* bw = A.bw + uh * DK * DV;
#pragma unroll
  for (int ct = 0; ct < DV / 16; ++ct) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) acc = F::mma(F::acc2(Z[2 * s], Z[2 * s + 1]), F::ld_tr<DVP>(sm.u.dO, 16 * ct, s, l16, kg), acc);
    store4<bf16>(bw + ((size_t)(w * (DV / 16) + ct) * 64 + lane) * 4, acc);
  }
}

// ---------------------------------------------------------------------------
// Step 3: the reverse state pass, per (sequence, head, 16*NWD-column slice;
// NWD = 4):
// dS_in = F^T dS_out + b = Diag(gam) dS_out - M^T dS_out + b, chunk by chunk
// from the last; the decay term in fp32, the correction on bf16 MFMA.  NWD wavefronts, one
// 16-column tile each.  F^T fragments are shared through LDS (double
// buffered); F^T and b are fetched NST chunks ahead into register stages
// used in turn (the loop is unrolled by NST).  The slices of a head read F^T
// through the same XCD's L2.
// ---------------------------------------------------------------------------
template <int DK, int DV, int NWD, int NST>
__global__ __launch_bounds__(64 * NWD) void chunk_bwd_dh_kernel(BwdArgs A) {
  constexpr int KS = DK / 32, KT = DK / 16, NTD = 64 * NWD, NS = DV / (16 * NWD);
  constexpr int FU = DK * DK / 8;     // 16-byte fragment units of F^T per chunk
  constexpr int FPT = FU / NTD;       // per thread
  static_assert(FPT * NTD == FU && NS * 16 * NWD == DV, "dh geometry");
  __shared__ u32x4 fbuf[2][FU];
  __shared__ float gbuf[2][DK];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the NS slices of a (sequence, head) share an XCD (and its L2)
  const int grp = blockIdx.x / (8 * NS), w8 = blockIdx.x % (8 * NS);
  const int unit = grp * 8 + (w8 & 7), slice = w8 >> 3;
  if (unit >= A.N * A.H) return;
  const int rank = unit / A.H, h = unit % A.H;
  const int n = A.cu_seqlens && A.order ? A.order[rank] : rank;
  const Seq sq = seq_info(A.cu_seqlens, n, A.T);
  const int nch = (sq.len + 63) / 64;
  const int slot0 = (sq.tok0 >> 6) + n;
  const int ct = slice * NWD + w;  // this wave's 16-column tile
  f32x4 ident;
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (4 * kg + i == l16) ? 1.f : 0.f;

  f32x4 dS[KT];
  {
    const float* d = A.dht ? A.dht + ((size_t)n * A.H + h) * DK * DV : nullptr;
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[mt][i] = d ? d[(size_t)(16 * mt + 4 * kg + i) * DV + 16 * ct + l16] : 0.f;
  }
  auto load_f = [&](u32x4 (&dst)[FPT], float& gdst, int cc) __attribute__((always_inline)) {
    const u32x4* p = reinterpret_cast<const u32x4*>(A.fw + ((size_t)(slot0 + cc) * A.H + h) * DK * DK);
#pragma unroll
    for (int j = 0; j < FPT; ++j) dst[j] = p[tid + NTD * j];
    gdst = tid < DK ? A.gw[((size_t)(slot0 + cc) * A.H + h) * DK + tid] : 0.f;
  };
  auto load_b = [&](bf16x4 (&dst)[KT], int cc) __attribute__((always_inline)) {
    const bf16* p = A.bw + ((size_t)(slot0 + cc) * A.H + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
      dst[mt] = __builtin_bit_cast(bf16x4, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
                                               p + ((size_t)(mt * (DV / 16) + ct) * 64 + lane) * 4)));
  };
  auto put_f = [&](const u32x4 (&src)[FPT], float gsrc, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FPT; ++j) fbuf[buf][tid + NTD * j] = src[j];
    if (tid < DK) gbuf[buf][tid] = gsrc;
  };
  // Register stages, used in turn: at iteration j (chunk cc = nch - 1 - j)
  // stage u = j % NST holds b of chunk cc and F^T of chunk cc - 1.  Both are
  // refilled in the same iteration (b with chunk cc - NST, F^T with chunk
  // cc - 1 - NST), so each load has NST iterations to land.  The refills are
  // unconditional (an index below zero rereads chunk 0): no copy between
  // stages and no merge of loaded and unloaded values, either of which makes
  // the compiler wait for the loads just issued.
  u32x4 fs[NST][FPT];
  float gs[NST];
  bf16x4 bs[NST][KT];
  auto step = [&](int cc, auto Uc) __attribute__((always_inline)) {
    constexpr int u = decltype(Uc)::value;
    __syncthreads();  // F^T of chunk cc is in fbuf[cc & 1]
    bf16* dh = A.dh + ((size_t)(slot0 + cc) * A.H + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
      store4<bf16>(dh + tile_off<DV>(16 * mt + l16, 16 * ct + 4 * kg), Reg16<bf16>::prod(dS[mt], ident));
    FV SF[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) SF[s] = F::acc2(dS[2 * s], dS[2 * s + 1]);
    const u32x4* fb = fbuf[cc & 1];
    const float* gb = gbuf[cc & 1];
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(&gb[16 * mt + 4 * kg]);
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = (float)bs[u][mt][i] + gm[i] * dS[mt][i];
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = F::mma(__builtin_bit_cast(FV, fb[(mt * KS + s) * 64 + lane]), SF[s], acc);
      dS[mt] = acc;
    }
    load_b(bs[u], max(cc - NST, 0));
    if (cc >= 1) put_f(fs[u], gs[u], (cc - 1) & 1);  // its buffer held chunk cc + 1, done before this iteration's barrier
    load_f(fs[u], gs[u], max(cc - 1 - NST, 0));
  };

  if (nch > 0) {
    load_f(fs[0], gs[0], nch - 1);
    put_f(fs[0], gs[0], (nch - 1) & 1);
    static_for<NST>([&](auto Uc) __attribute__((always_inline)) {
      constexpr int u = decltype(Uc)::value;
      load_b(bs[u], max(nch - 1 - u, 0));
      load_f(fs[u], gs[u], max(nch - 2 - u, 0));
    });
  }
  // whole groups of NST iterations, then the rest
  int j0 = 0;
  for (; j0 + NST <= nch; j0 += NST) static_for<NST>([&](auto Uc) __attribute__((always_inline)) { step(nch - 1 - j0 - decltype(Uc)::value, Uc); });
  static_for<NST>([&](auto Uc) __attribute__((always_inline)) {
    if (j0 + decltype(Uc)::value < nch) step(nch - 1 - j0 - decltype(Uc)::value, Uc);
  });
  // dh0 (fp32); for an empty sequence it is dht
  if (A.dh0) {
    float* d0 = A.dh0 + ((size_t)n * A.H + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) d0[(size_t)(16 * mt + 4 * kg + i) * DV + 16 * ct + l16] = dS[mt][i];
  }
}

// ---------------------------------------------------------------------------
// Step 4: per chunk-head, the chunk-local gradients.  Wave w owns key-channel
// tile w of the [DK][C] results; the [C][32] slice products and the [C][C]
// tiles are spread over the waves.
// ---------------------------------------------------------------------------
template <class Cfg>
struct LocalSmem {
  static constexpr int C = Cfg::C, DK = Cfg::DK, SP = Cfg::SP, CTP = Cfg::CTP;
  struct Slice {
    bf16 S[DK * SP], dS[DK * SP];  // S and Diag(gam) dS_out, value slice (rows: key channels)
    bf16 dO[C * SP], R[C * SP], U[C * SP], dU[C * SP], dR[C * SP];
  };
  struct Grads {
    bf16 dM[C * CTP], dP[C * CTP], dB[C * CTP], Y[C * CTP];
  };
  union {
    struct {
      FrontTiles<Cfg> ft;
      union {
        FrontScratch<Cfg> fs;
        Slice sl;
        Grads cc;
      } u;
    } m;
    float fin[4][C][DK + 4];  // dQt, dKt, dKh' (= dB^T Kt + dP^T Qt), dKb; token-major
  };
  alignas(16) float dgc[DK];     // rowsum(S * Diag(gam) dS_out)
  alignas(16) float dbt[4][C];   // dbeta partials from dT, by row block
  alignas(16) float dba[4][C];   // dbeta partials from dA, by column block
  alignas(16) float bsum[Cfg::NB][DK];
};

__device__ __forceinline__ void bstore_bf16(float v, rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)v), r, off, 0, 0);
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void chunk_bwd_local_kernel(BwdArgs A) {
  constexpr int DK = Cfg::DK, DV = Cfg::DV, GG = Cfg::GG, C = Cfg::C, KHP = Cfg::KHP, CTP = Cfg::CTP;
  constexpr int SP = Cfg::SP, VSL = Cfg::VSL, NW = Cfg::NW, NT = Cfg::NT, TB = Cfg::TB, NB = Cfg::NB;
  constexpr int SK = DK / 32;
  constexpr int MT = (20 + NW - 1) / NW;  // dP and dT tiles per wave
  static_assert(sizeof(LocalSmem<Cfg>) <= 163840, "LDS");
  __shared__ LocalSmem<Cfg> sm;
  const int H = A.H;
  const int h = blockIdx.x % H, slot = blockIdx.x / H;
  Seq sq;
  int c;
  if (!slot_chunk(A.cu_seqlens, A.N, A.T, slot, sq, c)) return;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x4 ident;
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (4 * kg + i == l16) ? 1.f : 0.f;
  for (int i = tid; i < 4 * C; i += NT) {
    (&sm.dbt[0][0])[i] = 0.f;
    (&sm.dba[0][0])[i] = 0.f;
  }
  const int nv = min(C, sq.len - c * C);
  const size_t row0 = (size_t)(sq.tok0 + c * C) * H + h;
  const int rsv = H * DV * 2;
  const rsrc_t bo = make_rsrc(A.dout + row0 * DV, (nv - 1) * rsv + DV * 2);
  const rsrc_t bv = make_rsrc(A.v + row0 * DV, (nv - 1) * rsv + DV * 2);
  const rsrc_t bdv = make_rsrc(A.dv + row0 * DV, (nv - 1) * rsv + DV * 2);
  const size_t uh = (size_t)slot * H + h;
  const bf16* hsS = A.hs + uh * DK * DV;
  const bf16* dhS = A.dh + uh * DK * DV;
  // The next value slice is fetched into registers one slice ahead (the
  // first one before the front): S and dS_out, one 8-element piece per
  // thread; dO (first 4C threads); V rows of this wave's R tiles.
  constexpr int NJ = 8 / NW;
  const int pr = tid >> 2, pp8 = 8 * (tid & 3);
  u32x4 s8, o8 = {0u, 0u, 0u, 0u};
  bf16x8 d8;
  bf16x4 vr[NJ];
  auto load_slice = [&](int v0) {
    s8 = *reinterpret_cast<const u32x4*>(hsS + tile_off<DV>(pr, v0 + pp8));
    d8 = *reinterpret_cast<const bf16x8*>(dhS + tile_off<DV>(pr, v0 + pp8));
    if (tid < 4 * C) o8 = bload<u32x4>(bo, pr * rsv + (v0 + pp8) * 2);
  };
  auto load_v = [&](int v0) {
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int job = w + NW * jj, tt = job >> 1, ct = job & 1;
      vr[jj] = bload<bf16x4>(bv, (16 * tt + l16) * rsv + (v0 + 16 * ct + 4 * kg) * 2);
    }
  };
  load_slice(0);
  load_v(0);

  float offref, mref, glref;
  FrontTiles<Cfg>& ft = sm.m.ft;
  {
    float G2f[TB];  // recomputed in the final stage (not kept live across the slices)
    chunk_front<Cfg, true>(A, sq, h, c, ft, sm.m.u.fs, G2f, offref, mref, glref, ident);
  }
  auto& sl = sm.m.u.sl;
  auto& cc = sm.m.u.cc;

  f32x4 cacc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) cacc[m] = zero4();
  f32x4 dQtT[4], SdR[4], dKbT[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) dQtT[tt] = SdR[tt] = dKbT[tt] = zero4();
  float rs = 0.f;  // rowsum(S * dS_out): channel 16w + l16, columns 8kg .. 8kg + 7 of each slice
  // the chunk-start Kt = kt e^{m} and chunk-end Kb = kh e^{G_last - m} row
  // fragments of this wave's R / dU tiles, the same for every value slice
  FV ktS[NJ][SK], kbS[NJ][SK];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int tt = (w + NW * jj) >> 1;
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      f32x4 lo, hi;
      row_vals(ft.em[tt], s, kg, lo, hi);
      ktS[jj][s] = scale8(ld_row<KHP>(ft.kt, 16 * tt + l16, s, kg), lo, hi);
      row_vals(ft.eb[tt], s, kg, lo, hi);
      kbS[jj][s] = scale8(ld_row<KHP>(ft.kh, 16 * tt + l16, s, kg), lo, hi);
    }
  }

  for (int v0 = 0; v0 < DV; v0 += VSL) {
    __syncthreads();  // the front, or the previous slice, is done with the slice tiles
    {
      // S and dS_out; dO
      const int r = pr, p8 = pp8;
      *reinterpret_cast<u32x2*>(&sl.S[r * SP + swz(r, p8)]) = u32x2{s8[0], s8[1]};
      *reinterpret_cast<u32x2*>(&sl.S[r * SP + swz(r, p8 + 4)]) = u32x2{s8[2], s8[3]};
      const u32x4 d4 = __builtin_bit_cast(u32x4, d8);
      *reinterpret_cast<u32x2*>(&sl.dS[r * SP + swz(r, p8)]) = u32x2{d4[0], d4[1]};
      *reinterpret_cast<u32x2*>(&sl.dS[r * SP + swz(r, p8 + 4)]) = u32x2{d4[2], d4[3]};
      if (tid < 4 * C) {
        *reinterpret_cast<u32x2*>(&sl.dO[r * SP + swz(r, p8)]) = u32x2{o8[0], o8[1]};
        *reinterpret_cast<u32x2*>(&sl.dO[r * SP + swz(r, p8 + 4)]) = u32x2{o8[2], o8[3]};
      }
    }
    if (v0 + VSL < DV) load_slice(v0 + VSL);
    __syncthreads();
    // R = V - Kt S and dU = Kh dSt + P^T dO = Kb dS_out + P^T dO (independent
    // of each other), with the chunk-start Kt = kt e^{m} and the chunk-end
    // Kb = kh e^{G_last - m} of the block-referenced rows
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int job = w + NW * jj, tt = job >> 1, ct = job & 1;
      f32x4 acc = zero4(), du = zero4();
#pragma unroll
      for (int s = 0; s < SK; ++s) acc = F::mma(ktS[jj][s], F::ld_tr<SP>(sl.S, 16 * ct, s, l16, kg), acc);
      st_acc<SP>(sl.R, 16 * tt, 16 * ct, Reg16<bf16>::rows(vr[jj], ident, -acc), ident, l16, kg);
#pragma unroll
      for (int s = 0; s < SK; ++s) du = F::mma(kbS[jj][s], F::ld_tr<SP>(sl.dS, 16 * ct, s, l16, kg), du);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (32 * s + 31 >= 16 * tt)
          du = F::mma(ld_row<CTP>(ft.u2, 16 * tt + l16, s, kg), F::ld_tr<SP>(sl.dO, 16 * ct, s, l16, kg), du);
      st_acc<SP>(sl.dU, 16 * tt, 16 * ct, du, ident, l16, kg);
    }
    if (v0 + VSL < DV) load_v(v0 + VSL);
    __syncthreads();
    // U = T R and dR = T^T dU, the value gradient
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int job = w + NW * jj, tt = job >> 1, ct = job & 1;
      f32x4 u = zero4(), dr = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (32 * s <= 16 * tt + 15)
          u = F::mma(ld_row<CTP>(ft.t, 16 * tt + l16, s, kg), F::ld_tr<SP>(sl.R, 16 * ct, s, l16, kg), u);
        if (32 * s + 31 >= 16 * tt)
          dr = F::mma(ld_row<CTP>(ft.u1, 16 * tt + l16, s, kg), F::ld_tr<SP>(sl.dU, 16 * ct, s, l16, kg), dr);
      }
      st_acc<SP>(sl.U, 16 * tt, 16 * ct, u, ident, l16, kg);
      const f32x4 rt = Reg16<bf16>::prod(dr, ident);  // rows of four columns
      st_row4<SP>(sl.dR, 16 * tt + l16, 16 * ct + 4 * kg, rt);
      bstore4(rt, bdv, (16 * tt + l16) * rsv + (v0 + 16 * ct + 4 * kg) * 2, bf16());
    }
    __syncthreads();
    // products over the slice's value columns
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int j = w + NW * m;
      if (j < 20) {
        int I, J;
        lower_tile(j % 10, I, J);
        const bf16* a = j < 10 ? sl.dO : sl.dU;
        const bf16* b = j < 10 ? sl.U : sl.R;
        cacc[m] = F::mma(ld_row<SP>(a, 16 * I + l16, 0, kg), ld_row<SP>(b, 16 * J + l16, 0, kg), cacc[m]);
      }
    }
    {
      const FV srow = ld_row<SP>(sl.S, 16 * w + l16, 0, kg);
      const FV drow = ld_row<SP>(sl.dS, 16 * w + l16, 0, kg);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        dQtT[tt] = F::mma(srow, ld_row<SP>(sl.dO, 16 * tt + l16, 0, kg), dQtT[tt]);
        SdR[tt] = F::mma(srow, ld_row<SP>(sl.dR, 16 * tt + l16, 0, kg), SdR[tt]);
        dKbT[tt] = F::mma(drow, ld_row<SP>(sl.U, 16 * tt + l16, 0, kg), dKbT[tt]);
      }
      const int r = 16 * w + l16;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int o = r * SP + swz(r, 8 * kg + 4 * e);
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(&sl.S[o]);
        const bf16x4 b = *reinterpret_cast<const bf16x4*>(&sl.dS[o]);
#pragma unroll
        for (int i = 0; i < 4; ++i) rs += (float)a[i] * (float)b[i];
      }
    }
  }
  // q, k of the final stage (thread = key channel, block of 16 tokens),
  // fetched now so that the loads overlap the C x C stage
  const int ch = tid % DK, tb = tid / DK;
  const int rsk = H * DK * 2, rsg = H * (DK / GG) * 2, rsb = H * 2;
  bf16 qf[TB], kf[TB], gf[TB];
  {
    const rsrc_t bq = make_rsrc(A.q + row0 * DK, (nv - 1) * rsk + DK * 2);
    const rsrc_t bk = make_rsrc(A.k + row0 * DK, (nv - 1) * rsk + DK * 2);
    const rsrc_t bg = make_rsrc(A.g + row0 * (DK / GG), (nv - 1) * rsg + (DK / GG) * 2);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      qf[j] = bload<bf16>(bq, (tb * TB + j) * rsk + ch * 2);
      kf[j] = bload<bf16>(bk, (tb * TB + j) * rsk + ch * 2);
      gf[j] = bload<bf16>(bg, (tb * TB + j) * rsg + (ch / GG) * 2);
    }
  }
  rs = rows4_sum(rs);
  if (kg == 0) sm.dgc[16 * w + l16] = rs * ft.gam[16 * w + l16];
  __syncthreads();  // slice tiles are free: the C x C gradient tiles take their place

  // zero the C x C gradient tiles (their zero blocks are never written)
  for (int i = tid; i < 4 * C * CTP / 4; i += NT) *reinterpret_cast<u32x2*>(&cc.dM[4 * i]) = u32x2{0u, 0u};
  __syncthreads();
  // dP, dT: masks; dbeta from T = X Diag(b); dM = dT Diag(b)
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int j = w + NW * m;
    if (j < 20) {
      int I, J;
      lower_tile(j % 10, I, J);
      f32x4 x = cacc[m];
      if (I == J) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = l16 <= 4 * kg + i ? x[i] : 0.f;
      }
      if (j < 10) {
        st_acc<CTP>(cc.dP, 16 * I, 16 * J, x, ident, l16, kg);
      } else {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * kg + i;
          part += x[i] * (float)ft.x[r * CTP + swz(r, 16 * J + l16)];
        }
        part = rows4_sum(part);
        if (kg == 0) sm.dbt[I][16 * J + l16] = part;
        st_acc<CTP>(cc.dM, 16 * I, 16 * J, x * ft.beta[16 * J + l16], ident, l16, kg);
      }
    }
  }
  __syncthreads();
  // Y = X^T dM
  for (int j = w; j < 16; j += NW) {
    const int I = j >> 2, J = j & 3, mx = I > J ? I : J;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (32 * s + 31 >= 16 * mx)
        acc = F::mma(F::ld_tr<CTP>(ft.x, 16 * I, s, l16, kg), F::ld_tr<CTP>(cc.dM, 16 * J, s, l16, kg), acc);
    st_acc<CTP>(cc.Y, 16 * I, 16 * J, acc, ident, l16, kg);
  }
  __syncthreads();
  // dA = -strict_lower(Y X^T); dbeta from A = Diag(b) B; dB = Diag(b) dA.
  // With eight wavefronts the six blocks below the diagonal (which carry the
  // reference shifts) go one to a wavefront and the four cheaper diagonal
  // blocks two to a wavefront; otherwise round-robin.
  const int na = NW == 8 ? (w < 6 ? 1 : 2) : (10 - w + NW - 1) / NW;
  for (int e = 0; e < na; ++e) {
    const int j = NW == 8 ? (w < 6 ? 4 + w : (e == 0 ? w - 6 : 9 - w)) : w + NW * e;
    int I, J;
    lower_tile(j, I, J);
    f32x4 acc = zero4(), bm = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (32 * s <= 16 * J + 15)
        acc = F::mma(ld_row<CTP>(cc.Y, 16 * I + l16, s, kg), ld_row<CTP>(ft.x, 16 * J + l16, s, kg), acc);
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      FV kt = ld_row<KHP>(ft.kt, 16 * I + l16, s, kg);
      if (I != J) {
        f32x4 lo, hi;
        row_shift(ft.gsum[I], ft.gsum[J], s, kg, lo, hi);
        kt = scale8(kt, lo, hi);
      }
      bm = F::mma(kt, ld_row<KHP>(ft.kh, 16 * J + l16, s, kg), bm);
    }
    f32x4 dA = -acc, pr = dA * bm;
    if (I == J) {
      // strictly lower part only; the upper part of a diagonal B tile holds
      // e^{G_i - G_j} with G_i > G_j, which may overflow: select, not scale
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool lower = l16 < 4 * kg + i;
        dA[i] = lower ? dA[i] : 0.f;
        pr[i] = lower ? pr[i] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = row_sum<16>(pr[i]);
    if (l16 == 0) *reinterpret_cast<f32x4*>(&sm.dba[J][16 * I + 4 * kg]) = pr;
    const f32x4 br = *reinterpret_cast<const f32x4*>(&ft.beta[16 * I + 4 * kg]);
    st_acc<CTP>(cc.dB, 16 * I, 16 * J, dA * br, ident, l16, kg);
  }
  __syncthreads();
  // the [DK][C] results of wave w, as gradients of the block-referenced tiles
  // (row channel 16w + 4kg + i, column token 16tt + l16): the state terms
  // carry e^{m} of the token's block; a pair of blocks (I, J) contributes
  // through its reference shift e^{m_I - m_J} (zero for I < J, where the
  // masked tiles vanish), applied to the transposed operand of lane channel
  // 16w + l16 whose elements 0..3 and 4..7 lie in blocks 2s and 2s + 1
  const int cw = 16 * w + l16;
  float mw[4], sh[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b) mw[b] = ft.gsum[b][cw];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int J = 0; J < 4; ++J) sh[I][J] = I > J ? fast_exp2(mw[I] - mw[J]) : (I == J ? 1.f : 0.f);
  auto shift = [&](int I, int J) { return sh[I][J]; };
  f32x4 dKtT[4], dKhT[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const f32x4 emr = *reinterpret_cast<const f32x4*>(&ft.em[tt][16 * w + 4 * kg]);
    dQtT[tt] *= emr;
    dKtT[tt] = -SdR[tt] * emr;
    dKhT[tt] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const FV khT = scale8(F::ld_tr<KHP>(ft.kh, 16 * w, s, l16, kg), splat4(shift(tt, 2 * s)),
                            splat4(shift(tt, 2 * s + 1)));
      dQtT[tt] = F::mma(khT, ld_row<CTP>(cc.dP, 16 * tt + l16, s, kg), dQtT[tt]);
      dKtT[tt] = F::mma(khT, ld_row<CTP>(cc.dB, 16 * tt + l16, s, kg), dKtT[tt]);
      const f32x4 lo = splat4(shift(2 * s, tt)), hi = splat4(shift(2 * s + 1, tt));
      dKhT[tt] = F::mma(scale8(F::ld_tr<KHP>(ft.kt, 16 * w, s, l16, kg), lo, hi),
                        F::ld_tr<CTP>(cc.dB, 16 * tt, s, l16, kg), dKhT[tt]);
      dKhT[tt] = F::mma(scale8(F::ld_tr<KHP>(ft.qt, 16 * w, s, l16, kg), lo, hi),
                        F::ld_tr<CTP>(cc.dP, 16 * tt, s, l16, kg), dKhT[tt]);
    }
  }
  __syncthreads();  // every tile is consumed: the final stage reuses the space
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int r = 16 * tt + l16, c0 = 16 * w + 4 * kg;
    *reinterpret_cast<f32x4*>(&sm.fin[0][r][c0]) = dQtT[tt];
    *reinterpret_cast<f32x4*>(&sm.fin[1][r][c0]) = dKtT[tt];
    *reinterpret_cast<f32x4*>(&sm.fin[2][r][c0]) = dKhT[tt];
    *reinterpret_cast<f32x4*>(&sm.fin[3][r][c0]) = dKbT[tt];
  }
  __syncthreads();

  // ---- final stage: thread = (key channel, block of 16 tokens) ----
  const rsrc_t bdq = make_rsrc(A.dq + row0 * DK, (nv - 1) * rsk + DK * 2);
  const rsrc_t bdk = make_rsrc(A.dk + row0 * DK, (nv - 1) * rsk + DK * 2);
  const rsrc_t bdg = make_rsrc(A.dg + row0 * (DK / GG), (nv - 1) * rsg + (DK / GG) * 2);
  // the chunk-start cumulative decay of this thread's tokens (log2 units),
  // formed exactly as the front formed it
  const float ebref = fast_exp2(glref - mref);
  float G2[TB];
  {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      acc += to_f32(gf[j]) * kLog2e;
      G2[j] = acc + offref;
    }
  }
  float dG[TB];
  float skb = 0.f;
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int r = tb * TB + j;
    const float dqt = sm.fin[0][r][ch], dkt = sm.fin[1][r][ch], dkh = sm.fin[2][r][ch], dkb = sm.fin[3][r][ch];
    // back from the block reference m and from the chunk end
    // e^{G_last - G} = e^{G_last - m} e^{m - G}: where the first factor
    // underflows the product is below e^-17 of the terms it joins
    const float eu = fast_exp2(G2[j] - mref), ed = fast_exp2(mref - G2[j]), ee = ebref * ed;
    const float q = to_f32(qf[j]), kk = to_f32(kf[j]);
    const float dq = dqt * eu, a = dkt * eu, kbe = dkb * ee, b = dkh * ed + kbe;
    dG[j] = q * dq + kk * (a - b);
    skb += kbe * kk;
    bstore_bf16(dq, bdq, r * rsk + ch * 2);
    bstore_bf16(a + b, bdk, r * rsk + ch * 2);
  }
  // reverse cumulative sum over the chunk; the chunk-total terms enter at
  // the last row and so reach every row
  float suf = 0.f;
#pragma unroll
  for (int j = TB - 1; j >= 0; --j) {
    suf += dG[j];
    dG[j] = suf;
  }
  sm.bsum[tb][ch] = skb;
  __syncthreads();
  float later = sm.dgc[ch];
#pragma unroll
  for (int b = 0; b < NB; ++b) later += sm.bsum[b][ch];
  __syncthreads();
  sm.bsum[tb][ch] = suf;
  __syncthreads();
  for (int b = tb + 1; b < NB; ++b) later += sm.bsum[b][ch];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int r = tb * TB + j;
    float x = dG[j] + later;
    if constexpr (GG == 1) {
      bstore_bf16(x, bdg, r * rsg + ch * 2);
    } else {
      x = rows4_sum(row_sum<16>(x));
      if (lane == 0) bstore_bf16(x, bdg, r * rsg + (ch / GG) * 2);
    }
  }
  if (tid < C) {
    float db = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) db += sm.dbt[b][tid];
#pragma unroll
    for (int b = 0; b < 4; ++b) db += sm.dba[b][tid];
    const rsrc_t bdb = make_rsrc(A.dbeta + row0, (nv - 1) * rsb + 2);
    bstore_bf16(db, bdb, tid * rsb);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <int DK, int DV, int GG>
static hipError_t launch_bwd_cfg(const BwdArgs& a, hipStream_t s) {
  typedef BwdCfg<DK, DV, GG> Cfg;
  const long long grid = (long long)a.slots * a.H;
  if (grid > 0) {
    hipLaunchKernelGGL(chunk_bwd_prep_kernel<Cfg>, dim3((unsigned)grid), dim3(Cfg::NT), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int units = a.N * a.H;
  if (units > 0) {
    constexpr int NWD = KDA_BWD_DH_WAVES;
    const int grid2 = (units + 7) / 8 * 8 * (DV / (16 * NWD));
    hipLaunchKernelGGL((chunk_bwd_dh_kernel<DK, DV, NWD, KDA_BWD_DH_STAGES>), dim3(grid2), dim3(64 * NWD), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (grid > 0) {
    hipLaunchKernelGGL(chunk_bwd_local_kernel<Cfg>, dim3((unsigned)grid), dim3(Cfg::NT), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int GG>
static hipError_t launch_bwd_g(int Dk, int Dv, const BwdArgs& a, hipStream_t s) {
  if (Dk == 64 && Dv == 64) return launch_bwd_cfg<64, 64, GG>(a, s);
  if (Dk == 64 && Dv == 128) return launch_bwd_cfg<64, 128, GG>(a, s);
  if (Dk == 128 && Dv == 64) return launch_bwd_cfg<128, 64, GG>(a, s);
  if (Dk == 128 && Dv == 128) return launch_bwd_cfg<128, 128, GG>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd(int Dk, int Dv, int g_group, const BwdArgs& a, hipStream_t s) {
  return g_group == 1 ? launch_bwd_g<1>(Dk, Dv, a, s) : launch_bwd_g<64>(Dk, Dv, a, s);
}

}  // namespace kda
