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
//   gated operands   Qt = Q*e^G, Kt = K*e^G, Kh = K*e^-G
//   k-k block        A  = strictly_lower(Diag(b) Kt Kh^T)              (MFMA)
//   q-k block        P  = lower_incl_diag(Qt Kh^T)                      (MFMA)
//   UT transform     Tm = (I + A)^-1 Diag(b): 16x16 diagonal blocks by a
//                    product of Neumann factors, the blocks below them by
//                    block forward substitution                         (MFMA)
//   state pass       R = V - Kt S;  U = Tm R;  O = Qt S + P U;
//                    S <- Diag(e^G_C) (S + Kh^T U)                      (MFMA)
//
// Design for MI355X.  The whole chain for one chunk runs in one workgroup and
// hands over through LDS, never through HBM: q, k, v, g, beta are read once
// and o written once.  A workgroup owns one (sequence, head, d_v slice) and
// walks that sequence's chunks in order.  Its wavefronts are specialised:
// producer wavefronts (one per 16 key channels) prepare chunk c -- gating,
// the k-k and q-k blocks, the UT transform -- while state wavefronts (one per
// 16 value columns of the slice, at most four) keep their columns of the fp32
// state in MFMA accumulators and run the state pass, which trails the
// producer by half a chunk.  The slices of one head are placed on the same
// XCD so that their shared q/k/g reads hit that XCD's L2.  bf16 inputs use
// v_mfma_f32_16x16x32_bf16 (fp32 accumulate); float32 inputs use
// v_mfma_f32_16x16x4_f32 throughout.
//
// Numerics: S, A, the diagonal solve, all accumulators and e^G are fp32; MFMA
// operands (gated q/k, Tm, P, R, U and a copy of S) are rounded to the input
// type.  Decay is referenced to the chunk start, so e^-G stays finite while a
// chunk's summed log-decay per channel is above about -80.

#include "kda_prefill_common.h"
#include "kda_launch.h"

namespace kda {

template <class Cfg>
struct Smem {
  typedef typename Cfg::E E;
  E q[Cfg::C][Cfg::KP];     // Qt = Q e^G          (token-major)
  E k[Cfg::C][Cfg::KP];     // Kt = K e^G          (token-major)
  E kh[Cfg::C][Cfg::KHP];   // Kh = K e^-G         (token-major; bf16: swizzled)
  E kht[Cfg::TR ? 1 : Cfg::DK][Cfg::CP];  // Kh^T  (fp32 only; key-channel-major, swizzled)
  E t[Cfg::C][Cfg::CP];     // Tm = (I + A)^-1 Diag(b), row-major
  E p[Cfg::C][Cfg::CP];     // P, row-major
  alignas(16) float a[Cfg::C][Cfg::AP];  // A (fp32), rows 16-byte aligned
  alignas(16) float xd[4][16][20];  // diagonal blocks of X = (I + A)^-1, row-major (fp32)
  alignas(16) float beta[Cfg::C];
  alignas(16) float gam[2][Cfg::DK];  // e^{G_C}, by chunk parity
  alignas(16) float gsum[Cfg::NPW][Cfg::DK];  // per-wavefront log2-decay totals
};


// ---------------------------------------------------------------------------
// The kernel.  Producer wavefronts prepare chunk c while state wavefronts run
// the state pass; one iteration, between LDS barriers:
//
//   X0 | producer: decay block sums, beta        | state: U = Tm R, O += P U, o
//  MID | producer: gated Qt, Kt, Kh, e^{G_C}     | state: S <- e^{G_C} (S + Kh^T U)
//   X1 | producer: A, P, diagonal solve blocks   | state: R = V - Kt S
//   X2 | producer: blocks below the diagonal, Kh^T | state: O = Qt S
//
// Each state wavefront owns TPW 16-column tiles of the slice and keeps S, R/U
// and O^T in registers; it reads V from HBM itself and producer outputs from
// LDS.  Products whose result leaves the registers are taken transposed
// (operands swapped), so that a lane holds four consecutive columns of a
// row: 8- or 16-byte writes to LDS and HBM.
// ---------------------------------------------------------------------------
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void chunk_fwd_kernel(PrefillArgs args) {
  typedef typename Cfg::T T;
  typedef typename Cfg::E E;
  typedef Frag<E> F;
  typedef typename F::V FV;
  constexpr int DK = Cfg::DK, DV = Cfg::DV, VS = Cfg::VS, GG = Cfg::GG, C = Cfg::C, KP = Cfg::KP;
  constexpr int NS = Cfg::NS, TPW = Cfg::TPW, KT = Cfg::KT, RPB = Cfg::RPB, NPW = Cfg::NPW;
  constexpr int SLAB = F::SLAB;
  constexpr int SK = DK / SLAB;  // slabs over key channels
  constexpr int SC = C / SLAB;   // slabs over the chunk's tokens

  __shared__ Smem<Cfg> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int l16 = lane & 15, kg = lane >> 4;
  const bool producer = wave < NPW;

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

  f32x4 ident;  // 16x16 identity, accumulator form
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (4 * kg + i == l16) ? 1.f : 0.f;

  // ---- upper 16x16 tiles of Tm and P are zero and never written again ----
  for (int idx = tid; idx < C * C; idx += Cfg::NT) {
    const int r = idx / C, c = idx % C;
    if ((c >> 4) > (r >> 4)) {
      sm.t[r][c] = from_f32<E>(0.f);
      sm.p[r][c] = from_f32<E>(0.f);
    }
  }

  // Fragments of the 16-row block blk of a token-major operand tile.
  auto ld_rows = [&](FV (&fr)[SK], const E (*tile)[KP], int blk) {
    const E* row = &tile[0][0] + opaque(l16 * KP) + 16 * blk * KP;
#pragma unroll
    for (int s = 0; s < SK; ++s) fr[s] = F::ld(row, s, kg);
  };
  // Same for the Kh tile (bf16: its units are XOR-permuted by row / 4).
  auto ld_kh_rows = [&](FV (&fr)[SK], int blk) {
    const E* row = &sm.kh[0][0] + opaque(l16 * Cfg::KHP) + 16 * blk * Cfg::KHP;
    const int kgx = Cfg::TR ? kg ^ kh_swizzle(l16) : kg;
#pragma unroll
    for (int s = 0; s < SK; ++s) fr[s] = F::ld(row, s, kgx);
  };
  auto mma_rows = [&](const FV (&a)[SK], const FV (&b)[SK]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SK; ++s) acc = F::mma(a[s], b[s], acc);
    return acc;
  };

  if (producer) {
    // ================= producer wavefronts ===================================
    // Gating map: thread = (8 key channels, block of RPB consecutive tokens);
    // the row blocks of one wavefront cover 64 / (DK / 8) * RPB consecutive tokens.
    typedef typename Vec8<T>::type V8;
    typedef typename Pair<E>::type EP2;
    constexpr int CGN = Cfg::CGN, RBW = Cfg::RBW;
    const int cg = tid % CGN, rb = tid / CGN;
    const int ch = 8 * cg;                 // first key channel of this thread
    const int rbw = lane / CGN;            // row block within the wavefront
    V8 rq[RPB], rk[RPB], rg[GG == 1 ? RPB : 1];
    T rgs[GG == 1 ? 1 : RPB], rbeta;
    // All loads of a chunk are in flight together; rows past the end of the
    // sequence read as zero through the per-chunk buffer bounds.
    const int rsk = H * DK * (int)sizeof(T);         // token stride of q, k (bytes)
    const int rsg = H * (DK / GG) * (int)sizeof(T);  // token stride of g
    const int rsb = H * (int)sizeof(T);              // token stride of beta
    // The prefetch of the next chunk is split in three parts, each issued as
    // soon as its registers are free, so that no single wave stalls on a long
    // burst of loads (the vector L1 moves about 64 bytes per clock).
    auto chunk_rows = [&](int ck) { return min(C, len - ck * C); };
    auto chunk_row0 = [&](int ck) { return (size_t)(tok0 + ck * C) * H + h; };
    auto load_gb = [&](int ck) {  // g, beta
      const int nv = chunk_rows(ck);
      const size_t row0 = chunk_row0(ck);
      const rsrc_t bg = make_rsrc(gg + row0 * (DK / GG), (nv - 1) * rsg + (DK / GG) * (int)sizeof(T));
      const rsrc_t bb = make_rsrc(gb + row0, (nv - 1) * rsb + (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) {
        const int r = rb * RPB + j;
        if constexpr (GG == 1)
          rg[j] = Vec8<T>::load(bg, r * rsg + ch * (int)sizeof(T));
        else
          rgs[j] = bload<T>(bg, r * rsg + (ch / GG) * (int)sizeof(T));
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
    EP2 khp[Cfg::TR ? 1 : 8][RPB / 2];  // fp32: Kh of this thread's rows per channel (token pairs), for Kh^T
    f32x4 Xdiag;            // X_ww = (I + A_ww)^-1 of this wave's block, accumulator form
    // Kh^T run of this thread: channels ch..ch+7 share one swizzle
    const int kht_col = ((((rb * RPB) >> 2) ^ kht_swizzle(ch)) << 2) | ((rb * RPB) & 3);

    // ---- tile jobs.  Operands are ordered for the transposed product, so a
    // lane ends with four consecutive columns of one row of the block. ----
    // A_IJ below the diagonal (I > J), fp32 row-major; khJ = fragments of Kh block J
    auto a_tile = [&](int I, int J, const FV (&khJ)[SK]) {
      FV kt[SK];
      ld_rows(kt, sm.k, I);
      const f32x4 d = mma_rows(khJ, kt) * sm.beta[opaque(l16) + 16 * I];
      *reinterpret_cast<f32x4*>(&sm.a[0][0] + opaque(l16 * Cfg::AP + 4 * kg) + 16 * I * Cfg::AP + 16 * J) = d;
    };
    // P_IJ below the diagonal (I > J)
    auto p_tile = [&](int I, int J, const FV (&khJ)[SK]) {
      FV qt[SK];
      ld_rows(qt, sm.q, I);
      store4<E>(&sm.p[0][0] + opaque(l16 * Cfg::CP + 4 * kg) + 16 * I * Cfg::CP + 16 * J, mma_rows(khJ, qt));
    };
    // Diagonal block I: N = A_II and N^T (registers only), P_II, and the
    // inverse X_II = (I + N)^-1 kept in registers for the forward substitution;
    // X_II (row-major, fp32) and Tm_II = X_II Diag(b_I) go to LDS.
    auto diag_job = [&](int I) {
      FV kt[SK], kh[SK], qt[SK];
      ld_rows(kt, sm.k, I);
      ld_kh_rows(kh, I);
      ld_rows(qt, sm.q, I);
      f32x4 N = mma_rows(kt, kh), Nt = mma_rows(kh, kt);
      f32x4 Pt = mma_rows(kh, qt);
      const float bl = sm.beta[opaque(l16) + 16 * I];
      const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[opaque(4 * kg) + 16 * I]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * kg + i;
        N[i] = l16 < r ? N[i] * br[i] : 0.f;  // strictly lower, rows scaled
        Nt[i] = r < l16 ? Nt[i] * bl : 0.f;
        Pt[i] = r <= l16 ? Pt[i] : 0.f;                     // lower including the diagonal
      }
      const int pt = opaque(l16 * Cfg::CP + 4 * kg) + 16 * I * Cfg::CP + 16 * I;
      store4<E>(&sm.p[0][0] + pt, Pt);
      Xdiag = unit_lower_inverse16<E>(N, Nt, ident);
      *reinterpret_cast<f32x4*>(&sm.xd[I][0][0] + opaque(20 * l16 + 4 * kg)) = Reg16<E>::prod(Xdiag, ident);
      store4<E>(&sm.t[0][0] + pt, Reg16<E>::prod(Xdiag * bl, ident));
    };
    // Blocks below the diagonal in block column J, top to bottom; each needs
    // only this column's blocks above it (registers) and the diagonal blocks:
    // X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ.
    auto solve_column = [&](auto Jc) {
      constexpr int J = decltype(Jc)::value;
      const float bj = sm.beta[opaque(l16) + 16 * J];
      const int ao = opaque(l16 * Cfg::AP + 4 * kg), xo = opaque(20 * l16 + 4 * kg);
      const int to = opaque(l16 * Cfg::CP + 4 * kg);
      f32x4 Xc[4 - J];  // X_KJ, K = J .. 3, accumulator form
      Xc[0] = Xdiag;
#pragma unroll
      for (int d = 1; d < 4 - J; ++d) {
        const int I = J + d;
        f32x4 M = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < d; ++e) {
          // (A_{I,J+e})^T in accumulator form: lane holds A[16I + l16][16(J+e) + 4kg + i]
          const f32x4 At = *reinterpret_cast<const f32x4*>(&sm.a[0][0] + ao + 16 * I * Cfg::AP + 16 * (J + e));
          M += Reg16<E>::prod(At, Xc[e]);
        }
        const f32x4 XIt = *reinterpret_cast<const f32x4*>(&sm.xd[I][0][0] + xo);
        Xc[d] = -Reg16<E>::prod(XIt, M);
        store4<E>(&sm.t[0][0] + to + 16 * I * Cfg::CP + 16 * J, Reg16<E>::prod(Xc[d] * bj, ident));
      }
    };

    if (nchunks > 0) {
      load_gb(0);
      load_q(0);
      load_k(0);
    }

    for (int it = 0; it <= nchunks; ++it) {
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
        if (tid < C) sm.beta[tid] = to_f32(rbeta);
      }
      lds_barrier();  // ------------------------------------------------- MID
      if (it + 1 < nchunks) load_gb(it + 1);  // prefetch (g, beta registers are free)
      if (it < nchunks) {
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
        // gated operands Qt, Kt, Kh (token-major)
        float eL[8];  // e^G of this thread's last row
#pragma unroll
        for (int j = 0; j < RPB; ++j) {
          const int r = rb * RPB + j;
          float e[8], n[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float Gc = off[c] + G[j][c];
            e[c] = fast_exp2(Gc);
            n[c] = fast_exp2(-Gc);
            if (j == RPB - 1) eL[c] = e[c];
          }
          float qo[8], ko[8], ho[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float kx = elem(rk[j], c);
            qo[c] = elem(rq[j], c) * e[c];
            ko[c] = kx * e[c];
            ho[c] = kx * n[c];
            if constexpr (!Cfg::TR) khp[c][j >> 1][j & 1] = from_f32<E>(ho[c]);
          }
#pragma unroll
          for (int c = 0; c < 8; c += 4) {
            store4<E>(&sm.q[r][ch + c], f32x4{qo[c], qo[c + 1], qo[c + 2], qo[c + 3]});
            store4<E>(&sm.k[r][ch + c], f32x4{ko[c], ko[c + 1], ko[c + 2], ko[c + 3]});
            const int khc = Cfg::TR ? 4 * (((ch + c) >> 2) ^ kh_swizzle(r)) : ch + c;
            store4<E>(&sm.kh[r][khc], f32x4{ho[c], ho[c + 1], ho[c + 2], ho[c + 3]});
          }
        }
        // the chunk's decay e^{G_C}: the last row of the chunk (its buffer
        // alternates with the chunk parity; the state pass reads the other)
        if (rb == Cfg::NRB - 1) {
          *reinterpret_cast<f32x4*>(&sm.gam[it & 1][ch]) = f32x4{eL[0], eL[1], eL[2], eL[3]};
          *reinterpret_cast<f32x4*>(&sm.gam[it & 1][ch + 4]) = f32x4{eL[4], eL[5], eL[6], eL[7]};
        }
      }
      lds_barrier();  // -------------------------------------------------- X1
      if (it + 1 < nchunks) load_q(it + 1);  // prefetch (q registers are free)
      if (it < nchunks) {
        // A and P: 10 + 10 tiles and four diagonal inverses over the producers
        static_switch<NPW>(wave, [&](auto Wc) {
          constexpr int W = decltype(Wc)::value;
          if constexpr (W < 4) diag_job(W);
          FV kh0[SK];
          if constexpr (NPW == 8) {
            if constexpr (W == 4) {
              ld_kh_rows(kh0, 0);
              a_tile(1, 0, kh0);
              p_tile(1, 0, kh0);
              a_tile(3, 0, kh0);
            } else if constexpr (W == 5) {
              ld_kh_rows(kh0, 0);
              p_tile(3, 0, kh0);
              a_tile(2, 0, kh0);
              p_tile(2, 0, kh0);
            } else if constexpr (W == 6) {
              ld_kh_rows(kh0, 1);
              a_tile(2, 1, kh0);
              p_tile(2, 1, kh0);
              a_tile(3, 1, kh0);
            } else if constexpr (W == 7) {
              ld_kh_rows(kh0, 1);
              p_tile(3, 1, kh0);
              ld_kh_rows(kh0, 2);
              a_tile(3, 2, kh0);
              p_tile(3, 2, kh0);
            }
          } else {  // four producers: the A blocks now, the P blocks with the solve
            if constexpr (W == 0) {
              ld_kh_rows(kh0, 0);
              a_tile(1, 0, kh0);
              a_tile(2, 0, kh0);
            } else if constexpr (W == 1) {
              ld_kh_rows(kh0, 1);
              a_tile(2, 1, kh0);
              ld_kh_rows(kh0, 0);
              a_tile(3, 0, kh0);
            } else if constexpr (W == 2) {
              ld_kh_rows(kh0, 1);
              a_tile(3, 1, kh0);
            } else if constexpr (W == 3) {
              ld_kh_rows(kh0, 2);
              a_tile(3, 2, kh0);
            }
          }
        });
      }
      lds_barrier();  // -------------------------------------------------- X2
      if (it + 1 < nchunks) load_k(it + 1);  // prefetch (k registers are free)
      if (it < nchunks) {
        static_switch<NPW>(wave, [&](auto Wc) {
          constexpr int W = decltype(Wc)::value;
          if constexpr (W < 3) solve_column(IC<W>{});
          if constexpr (NPW == 4 && W > 0) {  // P blocks below the diagonal, against the solve's load
            FV khj[SK];
#pragma unroll
            for (int J = 0; J < W; ++J) {
              ld_kh_rows(khj, J);
              p_tile(W, J, khj);
            }
          }
        });
        // fp32: transposed Kh, read by the state pass next
        if constexpr (!Cfg::TR) {
#pragma unroll
          for (int c = 0; c < 8; ++c) store_pairs<E, RPB / 2>(&sm.kht[ch + c][kht_col], khp[c]);
        }
      }
    }
    return;
  }

  // ================= state wavefronts ======================================
  const int bw = wave - NPW;  // state wavefront index
  // The state pass carries the recurrence; its short VALU/LDS/MFMA bursts are
  // issued ahead of the producers' long VALU streams on the same SIMD.
  __builtin_amdgcn_s_setprio(2);
  f32x4 S[TPW][KT];         // S: rows (key channels) 16mt + 4kg + i, column l16
  f32x4 R[TPW][4];          // R, then U: token rows 16t + 4kg + i, column l16
  f32x4 O[TPW][4];          // O^T: lane holds token 16t + l16, columns 4kg + i
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

  const int rsv = H * DV * (int)sizeof(T);  // token stride of v and o (bytes)
  // V rows of the next chunk: lane holds 4 columns of token 16t + l16
  typename Row4<T>::type vr[TPW][4];
  auto load_v = [&](int ck) {
    const int nv = min(C, len - ck * C);
    const rsrc_t bv = make_rsrc(gv + ((size_t)(tok0 + ck * C) * H + h) * DV + col0, (nv - 1) * rsv + VS * (int)sizeof(T));
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vr[j][t] = bload<typename Row4<T>::type>(bv, (16 * t + l16) * rsv + (16 * (TPW * bw + j) + 4 * kg) * (int)sizeof(T));
  };
  if (nchunks > 0) load_v(0);

  FV UF[TPW][SC];  // U as operand fragments (bf16 or fp32)
  for (int it = 0; it <= nchunks; ++it) {
    lds_barrier();  // -------------------------------------------------- X0
    if (it >= 1) {
      // ---- state: U = Tm R (Tm lower triangular: tile t needs k < 16(t+1)) ----
      {
        FV RF[TPW][SC];
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
            const FV a = F::ld(trow, s, kg);
#pragma unroll
            for (int j = 0; j < TPW; ++j) R[j][t] = F::mma(a, RF[j][s], R[j][t]);
          }
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int s = 0; s < SC; ++s) UF[j][s] = acc_frag(R[j], s, E());
      }
      // ---- O^T += U^T P^T, then write o of chunk it - 1 (rows of 4 columns) ----
      const int pbase = (it - 1) * C;
      const int nv = min(C, len - pbase);
      const rsrc_t bo = make_rsrc(go + ((size_t)(tok0 + pbase) * H + h) * DV + col0, (nv - 1) * rsv + VS * (int)sizeof(T));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const E* prow = &sm.p[16 * t + l16][0];
#pragma unroll
        for (int s = 0; s < (16 * (t + 1) + SLAB - 1) / SLAB; ++s) {
          const FV b = F::ld(prow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j][t] = F::mma(UF[j][s], b, O[j][t]);
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          bstore4(O[j][t], bo, (16 * t + l16) * rsv + (16 * (TPW * bw + j) + 4 * kg) * (int)sizeof(T), T());
      }
    }
    lds_barrier();  // ------------------------------------------------- MID
    if (it >= 1) {
      // ---- state: S <- Diag(e^{G_C}) (S + Kh^T U) ----
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        const E* krow = &sm.kht[Cfg::TR ? 0 : 16 * mt + l16][0];
        const int sw = kht_swizzle(16 * mt);
#pragma unroll
        for (int s = 0; s < SC; ++s) {
          FV a;
          if constexpr (Cfg::TR)
            a = F::template ld_tr<Cfg::KHP>(&sm.kh[0][0], 16 * mt, s, l16, kg);
          else
            a = F::ld_sw(krow, s, kg, sw);
#pragma unroll
          for (int j = 0; j < TPW; ++j) S[j][mt] = F::mma(a, UF[j][s], S[j][mt]);
        }
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gam[(it - 1) & 1][16 * mt + 4 * kg]);
#pragma unroll
        for (int j = 0; j < TPW; ++j) S[j][mt] *= gm;
      }
    }
    lds_barrier();  // -------------------------------------------------- X1
    if (it < nchunks) {
      // ---- state: R = V - Kt S (V enters through an exact identity product) ----
      FV SF[TPW][SK];  // -S as B-operand fragments
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int s = 0; s < SK; ++s) SF[j][s] = acc_frag_neg(S[j], s, E());
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) R[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const E* krow = &sm.k[16 * t + l16][0];
#pragma unroll
        for (int s = 0; s < SK; ++s) {
          const FV a = F::ld(krow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) R[j][t] = F::mma(a, SF[j][s], R[j][t]);
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) R[j][t] = Reg16<E>::rows(vr[j][t], ident, R[j][t]);
      }
      if (it + 1 < nchunks) load_v(it + 1);  // prefetch (V registers are free)
    }
    lds_barrier();  // -------------------------------------------------- X2
    if (it < nchunks) {
      // ---- state: O^T = S^T Qt^T ----
      FV SF[TPW][SK];
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
          const FV b = F::ld(qrow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j][t] = F::mma(SF[j][s], b, O[j][t]);
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
  KDA_CASE(64, 64, 32)
  KDA_CASE(64, 64, 16)
  KDA_CASE(64, 128, 32)
  KDA_CASE(64, 128, 16)
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
  if (bf16_io) return launch_prefill_pipe(Dk, Dv, g_group, VS, a, stream);  // kda_prefill_pipe.hip
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

