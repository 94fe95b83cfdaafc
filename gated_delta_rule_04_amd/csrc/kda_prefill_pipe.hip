// KDA chunked prefill for bf16 inputs, gfx950: the producer work is
// software-pipelined across chunks.
//
// Same block algebra as the single-stage kernel (kda_prefill.hip): per chunk
// of C = 64 tokens the gated operands Qt = Q e^G, Kt = K e^G, Kh = K e^-G, the
// blocks A = strictly_lower(Diag(b) Kt Kh^T) and P = lower_incl_diag(Qt Kh^T),
// the UT transform Tm = (I + A)^-1 Diag(b), and the state pass R = V - Kt S,
// U = Tm R, O = Qt S + P U, S <- Diag(e^{G_C}) (S + Kh^T U).  It is derived
// from the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t
// v_t^T, o_t = S_t^T q_t of the miniKimiK3 card's Kimi Delta Attention bullet
// ("Architecture" section) and is exact up to rounding.
//
// Only the state pass is a recurrence; gating and the transform of a chunk
// depend on its own inputs alone.  Here they run ahead of the state pass, so
// that the VALU-bound gating of one chunk overlaps the MFMA- and
// latency-bound transform of the next and the state pass of the one after.
// Each iteration i has two stages between workgroup barriers:
//
//   stage | state wavefronts           | producers: transform | producers: gating
//   ------+----------------------------+----------------------+-------------------
//     P   | chunk i:   U = Tm R,       | chunk i+1: A, P,     | chunk i+2: decay
//         |   O += P U, o, S update    |   diagonal inverses  |   block sums, beta
//     Q   | chunk i+1: R = V - Kt S,   | chunk i+1: blocks    | chunk i+2: Qt, Kt,
//         |   O = Qt S                 |   below the diagonal |   Kh, e^{G_C}
//
// The gated operands, Tm, P, beta and e^{G_C} are double-buffered in LDS by
// chunk parity.  Kh^T fragments come from the token-major Kh tile through
// gfx950 transposing LDS reads, and A keeps only its six blocks below the
// diagonal, which is what makes the two buffers fit in 160 KB at d_k = 128.
// Global loads are issued one full iteration before their use.

#include "kda_prefill_common.h"
#include "kda_launch.h"

namespace kda {

template <class Cfg>
struct PipeSmem {
  typedef typename Cfg::E E;
  E q[2][Cfg::C][Cfg::KP];    // Qt = Q e^G          (token-major), by chunk parity
  E k[2][Cfg::C][Cfg::KP];    // Kt = K e^G          (token-major)
  E kh[2][Cfg::C][Cfg::KHP];  // Kh = K e^-G         (token-major, swizzled)
  E t[2][Cfg::C][Cfg::CP];    // Tm = (I + A)^-1 Diag(b), row-major
  E p[2][Cfg::C][Cfg::CP];    // P, row-major
  alignas(16) float a[6][16][20];   // blocks A_IJ, I > J (fp32), block I(I-1)/2 + J
  alignas(16) float xd[4][16][20];  // diagonal blocks of X = (I + A)^-1, row-major (fp32)
  alignas(16) float beta[2][Cfg::C];
  alignas(16) float gam[2][Cfg::DK];         // e^{G_C}
  alignas(16) float gsum[Cfg::NPW][Cfg::DK];  // per-wavefront log2-decay totals
};

template <class Cfg, bool PRO>
__global__ __launch_bounds__(Cfg::NT) void chunk_fwd_pipe_kernel(PrefillArgs args) {
  typedef typename Cfg::T T;
  typedef typename Cfg::E E;
  typedef Frag<E> F;
  typedef typename F::V FV;
  static_assert(Cfg::TR, "bf16 path");
  constexpr int DK = Cfg::DK, DV = Cfg::DV, VS = Cfg::VS, GG = Cfg::GG, C = Cfg::C, KP = Cfg::KP;
  constexpr int KHP = Cfg::KHP, CP = Cfg::CP;
  constexpr int NS = Cfg::NS, TPW = Cfg::TPW, KT = Cfg::KT, RPB = Cfg::RPB, NPW = Cfg::NPW;
  constexpr int SLAB = F::SLAB;
  constexpr int SK = DK / SLAB;  // slabs over key channels
  constexpr int SC = C / SLAB;   // slabs over the chunk's tokens

  __shared__ PipeSmem<Cfg> sm;

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
  // chunk c of this sequence keeps its entering state in slot hs_slot0 + c
  const int hs_slot0 = (tok0 >> 6) + seq;
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
  for (int idx = tid; idx < 2 * C * C; idx += Cfg::NT) {
    const int b = idx / (C * C), r = (idx / C) % C, c = idx % C;
    if ((c >> 4) > (r >> 4)) {
      sm.t[b][r][c] = from_f32<E>(0.f);
      sm.p[b][r][c] = from_f32<E>(0.f);
    }
  }

  // Fragments of the 16-row block blk of a token-major Qt or Kt tile.
  auto ld_rows = [&](FV (&fr)[SK], const E (*tile)[KP], int blk) {
    const E* row = &tile[0][0] + opaque(l16 * KP) + 16 * blk * KP;
#pragma unroll
    for (int s = 0; s < SK; ++s) fr[s] = F::ld(row, s, kg);
  };
  // Same for a Kh tile (its units are XOR-permuted by row / 4).
  auto ld_kh_rows = [&](FV (&fr)[SK], int b, int blk) {
    const E* row = &sm.kh[b][0][0] + opaque(l16 * KHP) + 16 * blk * KHP;
    const int kgx = kg ^ kh_swizzle(l16);
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
    // Gating map: thread = (8 key channels, block of RPB consecutive tokens).
    typedef typename Vec8<T>::type V8;
    constexpr int CGN = Cfg::CGN, RBW = Cfg::RBW;
    const int cg = tid % CGN, rb = tid / CGN;
    const int ch = 8 * cg;                 // first key channel of this thread
    const int rbw = lane / CGN;            // row block within the wavefront
    V8 rq[RPB], rk[RPB], rg[GG == 1 ? RPB : 1];
    T rgs[GG == 1 ? 1 : RPB], rbeta;
    // Rows past the end of the sequence read as zero through the per-chunk
    // buffer bounds.
    const int rsk = H * DK * (int)sizeof(T);         // token stride of q, k (bytes)
    const int rsg = H * (DK / GG) * (int)sizeof(T);  // token stride of g
    const int rsb = H * (int)sizeof(T);              // token stride of beta
    // prologue: -exp(A_log) and dt_bias log2(e) of this thread's channels (or group)
    constexpr int NGC = PRO ? (GG == 1 ? 8 : 1) : 1;
    float nA[NGC], gDs[NGC];
    if constexpr (PRO) {
#pragma unroll
      for (int c = 0; c < NGC; ++c) {
        const int gi = h * (DK / GG) + (GG == 1 ? ch + c : ch / GG);
        nA[c] = -fast_exp2(args.A_log[gi] * kLog2e);
        gDs[c] = args.dt_bias[gi] * kLog2e;
      }
    }
    // log2 of a decay from its gate: the gate itself, or under the prologue
    // -exp(A_log) softplus(g + dt_bias)
    auto lg_gate = [&](float x, int c) {
      if constexpr (PRO)
        return nA[c] * softplus_log2(fmaf(x, kLog2e, gDs[c]));
      else
        return x * kLog2e;
    };
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
    auto load_qk = [&](int ck) {
      const rsrc_t bq = make_rsrc(gq + chunk_row0(ck) * DK, (chunk_rows(ck) - 1) * rsk + DK * (int)sizeof(T));
      const rsrc_t bk = make_rsrc(gk + chunk_row0(ck) * DK, (chunk_rows(ck) - 1) * rsk + DK * (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) rq[j] = Vec8<T>::load(bq, (rb * RPB + j) * rsk + ch * (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) rk[j] = Vec8<T>::load(bk, (rb * RPB + j) * rsk + ch * (int)sizeof(T));
    };
    float G[RPB][8];  // cumulative log2-decay of this thread's rows (block-local)
    float off[8];     // log2-decay of the chunk before this thread's block
    f32x4 Xdiag;      // X_ww = (I + A_ww)^-1 of this wave's block, accumulator form

    // ---- transform jobs for the chunk in buffer b.  Operands are ordered for
    // the transposed product, so a lane ends with four consecutive columns of
    // one row of the block. ----
    // A_IJ below the diagonal (I > J), fp32; khJ = fragments of Kh block J
    auto a_tile = [&](int b, int I, int J, const FV (&khJ)[SK]) {
      FV kt[SK];
      ld_rows(kt, sm.k[b], I);
      const f32x4 d = mma_rows(khJ, kt) * sm.beta[b][opaque(l16) + 16 * I];
      *reinterpret_cast<f32x4*>(&sm.a[I * (I - 1) / 2 + J][0][0] + opaque(20 * l16 + 4 * kg)) = d;
    };
    // P_IJ below the diagonal (I > J)
    auto p_tile = [&](int b, int I, int J, const FV (&khJ)[SK]) {
      FV qt[SK];
      ld_rows(qt, sm.q[b], I);
      store4<E>(&sm.p[b][0][0] + opaque(l16 * CP + 4 * kg) + 16 * I * CP + 16 * J, mma_rows(khJ, qt));
    };
    // Diagonal block I: N = A_II and N^T (registers only), P_II, and the
    // inverse X_II = (I + N)^-1 kept in registers for the forward substitution;
    // X_II (row-major, fp32) and Tm_II = X_II Diag(b_I) go to LDS.
    auto diag_job = [&](int b, int I) {
      FV kt[SK], kh[SK], qt[SK];
      ld_rows(kt, sm.k[b], I);
      ld_kh_rows(kh, b, I);
      ld_rows(qt, sm.q[b], I);
      f32x4 N = mma_rows(kt, kh), Nt = mma_rows(kh, kt);
      f32x4 Pt = mma_rows(kh, qt);
      const float bl = sm.beta[b][opaque(l16) + 16 * I];
      const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[b][opaque(4 * kg) + 16 * I]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * kg + i;
        N[i] = l16 < r ? N[i] * br[i] : 0.f;  // strictly lower, rows scaled
        Nt[i] = r < l16 ? Nt[i] * bl : 0.f;
        Pt[i] = r <= l16 ? Pt[i] : 0.f;       // lower including the diagonal
      }
      const int pt = opaque(l16 * CP + 4 * kg) + 16 * I * CP + 16 * I;
      store4<E>(&sm.p[b][0][0] + pt, Pt);
      Xdiag = unit_lower_inverse16<E>(N, Nt, ident);
      *reinterpret_cast<f32x4*>(&sm.xd[I][0][0] + opaque(20 * l16 + 4 * kg)) = Reg16<E>::prod(Xdiag, ident);
      store4<E>(&sm.t[b][0][0] + pt, Reg16<E>::prod(Xdiag * bl, ident));
    };
    // Blocks below the diagonal in block column J, top to bottom; each needs
    // only this column's blocks above it (registers) and the diagonal blocks:
    // X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ.
    auto solve_column = [&](int b, auto Jc) {
      constexpr int J = decltype(Jc)::value;
      const float bj = sm.beta[b][opaque(l16) + 16 * J];
      const int ao = opaque(20 * l16 + 4 * kg), to = opaque(l16 * CP + 4 * kg);
      f32x4 Xc[4 - J];  // X_KJ, K = J .. 3, accumulator form
      Xc[0] = Xdiag;
#pragma unroll
      for (int d = 1; d < 4 - J; ++d) {
        const int I = J + d;
        f32x4 M = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < d; ++e) {
          // (A_{I,J+e})^T in accumulator form: lane holds A[16I + l16][16(J+e) + 4kg + i]
          const f32x4 At = *reinterpret_cast<const f32x4*>(&sm.a[I * (I - 1) / 2 + J + e][0][0] + ao);
          M += Reg16<E>::prod(At, Xc[e]);
        }
        const f32x4 XIt = *reinterpret_cast<const f32x4*>(&sm.xd[I][0][0] + ao);
        Xc[d] = -Reg16<E>::prod(XIt, M);
        store4<E>(&sm.t[b][0][0] + to + 16 * I * CP + 16 * J, Reg16<E>::prod(Xc[d] * bj, ident));
      }
    };

    if (nchunks > 0) {
      load_gb(0);
      load_qk(0);
    }

    for (int i = -2; i < nchunks; ++i) {
      const int cT = i + 1, cG = i + 2;  // chunks under transform and gating
      const int bT = cT & 1, bG = cG & 1;
      lds_barrier();  // ---------------------------------------------------- P
      if (cT >= 0 && cT < nchunks) {
        // A and P: 10 + 10 tiles and four diagonal inverses over the producers
        static_switch<NPW>(wave, [&](auto Wc) {
          constexpr int W = decltype(Wc)::value;
          if constexpr (W < 4) diag_job(bT, W);
          FV kh0[SK];
          if constexpr (NPW == 8) {
            if constexpr (W == 4) {
              ld_kh_rows(kh0, bT, 0);
              a_tile(bT, 1, 0, kh0);
              p_tile(bT, 1, 0, kh0);
              a_tile(bT, 3, 0, kh0);
            } else if constexpr (W == 5) {
              ld_kh_rows(kh0, bT, 0);
              p_tile(bT, 3, 0, kh0);
              a_tile(bT, 2, 0, kh0);
              p_tile(bT, 2, 0, kh0);
            } else if constexpr (W == 6) {
              ld_kh_rows(kh0, bT, 1);
              a_tile(bT, 2, 1, kh0);
              p_tile(bT, 2, 1, kh0);
              a_tile(bT, 3, 1, kh0);
            } else if constexpr (W == 7) {
              ld_kh_rows(kh0, bT, 1);
              p_tile(bT, 3, 1, kh0);
              ld_kh_rows(kh0, bT, 2);
              a_tile(bT, 3, 2, kh0);
              p_tile(bT, 3, 2, kh0);
            }
          } else {  // four producers: the A blocks now, the P blocks with the solve
            if constexpr (W == 0) {
              ld_kh_rows(kh0, bT, 0);
              a_tile(bT, 1, 0, kh0);
              a_tile(bT, 2, 0, kh0);
            } else if constexpr (W == 1) {
              ld_kh_rows(kh0, bT, 1);
              a_tile(bT, 2, 1, kh0);
              ld_kh_rows(kh0, bT, 0);
              a_tile(bT, 3, 0, kh0);
            } else if constexpr (W == 2) {
              ld_kh_rows(kh0, bT, 1);
              a_tile(bT, 3, 1, kh0);
            } else if constexpr (W == 3) {
              ld_kh_rows(kh0, bT, 2);
              a_tile(bT, 3, 2, kh0);
            }
          }
        });
      }
      if (cG < nchunks) {
        // block-local cumulative decay; prefix over this wavefront's blocks
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.f;
        // rows past the end of the sequence stay inert under the prologue too:
        // their (zero) gate logits must not become a decay.  A full chunk
        // (uniform test) skips the per-row mask.
        const int nvG = chunk_rows(cG);
        auto gate_rows = [&](auto Full) {
          constexpr bool FULL = decltype(Full)::value;
#pragma unroll
          for (int j = 0; j < RPB; ++j) {
            const bool live = FULL || rb * RPB + j < nvG;
            float lrow = 0.f;  // decay-group gate of row j (log2 units)
            if constexpr (GG != 1) {
              lrow = lg_gate(to_f32(rgs[j]), 0);
              if constexpr (!FULL) lrow = live ? lrow : 0.f;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              float lx = lrow;
              if constexpr (GG == 1) {
                lx = lg_gate(elem(rg[j], c), c);
                if constexpr (!FULL) lx = live ? lx : 0.f;
              }
              acc[c] += lx;
              G[j][c] = acc[c];
            }
          }
        };
        if (!PRO || nvG == C)
          gate_rows(IC<1>{});
        else
          gate_rows(IC<0>{});
        if constexpr (RBW == 4) {  // the four row blocks are the wavefront's 16-lane rows
          float tot[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) rows4_scan(acc[c], rbw, off[c], tot[c]);
          if (rbw == RBW - 1) {
            *reinterpret_cast<f32x4*>(&sm.gsum[wave][ch]) = f32x4{tot[0], tot[1], tot[2], tot[3]};
            *reinterpret_cast<f32x4*>(&sm.gsum[wave][ch + 4]) = f32x4{tot[4], tot[5], tot[6], tot[7]};
          }
        } else {
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
        }
        if (tid < C) sm.beta[bG][tid] = PRO ? (tid < nvG ? sigmoid_f(to_f32(rbeta)) : 0.f) : to_f32(rbeta);
        if (cG + 1 < nchunks) load_gb(cG + 1);  // prefetch (g, beta registers are free)
      }
      lds_barrier();  // ---------------------------------------------------- Q
      if (cT >= 0 && cT < nchunks) {
        static_switch<NPW>(wave, [&](auto Wc) {
          constexpr int W = decltype(Wc)::value;
          if constexpr (W < 3) solve_column(bT, IC<W>{});
          if constexpr (NPW == 4 && W > 0) {  // P blocks below the diagonal, against the solve's load
            FV khj[SK];
#pragma unroll
            for (int J = 0; J < W; ++J) {
              ld_kh_rows(khj, bT, J);
              p_tile(bT, W, J, khj);
            }
          }
        });
      }
      if (cG < nchunks) {
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
        // prologue: inverse L2 norms of this thread's q and k rows (a row's
        // channels are spread over CGN consecutive lanes)
        float iq[RPB], ik[RPB];
#pragma unroll
        for (int j = 0; j < RPB; ++j) iq[j] = ik[j] = 1.f;
        if constexpr (PRO) {
#pragma unroll
          for (int j = 0; j < RPB; ++j) {
            const float sq = row_sum<CGN>(sumsq8(rq[j]));
            const float sk = row_sum<CGN>(sumsq8(rk[j]));
            iq[j] = __builtin_amdgcn_rsqf(sq + kNormEps);
            ik[j] = __builtin_amdgcn_rsqf(sk + kNormEps);
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
            const float kx = elem(rk[j], c) * ik[j];
            qo[c] = elem(rq[j], c) * iq[j] * e[c];
            ko[c] = kx * e[c];
            ho[c] = kx * n[c];
          }
#pragma unroll
          for (int c = 0; c < 8; c += 4) {
            store4<E>(&sm.q[bG][r][ch + c], f32x4{qo[c], qo[c + 1], qo[c + 2], qo[c + 3]});
            store4<E>(&sm.k[bG][r][ch + c], f32x4{ko[c], ko[c + 1], ko[c + 2], ko[c + 3]});
            store4<E>(&sm.kh[bG][r][4 * (((ch + c) >> 2) ^ kh_swizzle(r))],
                      f32x4{ho[c], ho[c + 1], ho[c + 2], ho[c + 3]});
          }
        }
        // the chunk's decay e^{G_C}: the last row of the chunk
        if (rb == Cfg::NRB - 1) {
          *reinterpret_cast<f32x4*>(&sm.gam[bG][ch]) = f32x4{eL[0], eL[1], eL[2], eL[3]};
          *reinterpret_cast<f32x4*>(&sm.gam[bG][ch + 4]) = f32x4{eL[4], eL[5], eL[6], eL[7]};
        }
        if (cG + 1 < nchunks) load_qk(cG + 1);  // prefetch (q, k registers are free)
      }
    }
    return;
  }

  // ================= state wavefronts ======================================
  const int bw = wave - NPW;  // state wavefront index
  // The state pass carries the recurrence; its short VALU/LDS/MFMA bursts are
  // issued ahead of the producers' long VALU streams on the same SIMD.
  __builtin_amdgcn_s_setprio(2);
  f32x4 S[TPW][KT];  // S: rows (key channels) 16mt + 4kg + i, column l16
  f32x4 R[TPW][4];   // R, then U: token rows 16t + 4kg + i, column l16
  f32x4 O[TPW][4];   // O^T: lane holds token 16t + l16, columns 4kg + i
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

  for (int i = -2; i < nchunks; ++i) {
    lds_barrier();  // ------------------------------------------------------ P
    if (i >= 0) {
      const int b = i & 1;
      // ---- U = Tm R (Tm lower triangular: tile t needs k < 16(t+1)) ----
      FV UF[TPW][SC];  // U as operand fragments
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
          const E* trow = &sm.t[b][16 * t + l16][0];
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
      // ---- O^T += U^T P^T, then write o of chunk i (rows of 4 columns) ----
      const int nv = min(C, len - i * C);
      const rsrc_t bo = make_rsrc(go + ((size_t)(tok0 + i * C) * H + h) * DV + col0, (nv - 1) * rsv + VS * (int)sizeof(T));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const E* prow = &sm.p[b][16 * t + l16][0];
#pragma unroll
        for (int s = 0; s < (16 * (t + 1) + SLAB - 1) / SLAB; ++s) {
          const FV pb = F::ld(prow, s, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j][t] = F::mma(UF[j][s], pb, O[j][t]);
        }
        if (go) {
#pragma unroll
          for (int j = 0; j < TPW; ++j)
            bstore4(O[j][t], bo, (16 * t + l16) * rsv + (16 * (TPW * bw + j) + 4 * kg) * (int)sizeof(T), T());
        }
      }
      // ---- S <- Diag(e^{G_C}) (S + Kh^T U) ----
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
#pragma unroll
        for (int s = 0; s < SC; ++s) {
          const FV a = F::template ld_tr<KHP>(&sm.kh[b][0][0], 16 * mt, s, l16, kg);
#pragma unroll
          for (int j = 0; j < TPW; ++j) S[j][mt] = F::mma(a, UF[j][s], S[j][mt]);
        }
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gam[b][16 * mt + 4 * kg]);
#pragma unroll
        for (int j = 0; j < TPW; ++j) S[j][mt] *= gm;
      }
    }
    lds_barrier();  // ------------------------------------------------------ Q
    if (i + 1 >= 0 && i + 1 < nchunks) {
      const int b = (i + 1) & 1;
      // ---- optional: the state entering chunk i + 1, in the operand type
      // (rows of four columns through an exact transposing product) ----
      if (args.hs) {
        E* hs = static_cast<E*>(args.hs) + ((size_t)(hs_slot0 + i + 1) * H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int mt = 0; mt < KT; ++mt)
            store4<E>(hs + (size_t)(16 * mt + l16) * DV + col0 + 16 * (TPW * bw + j) + 4 * kg,
                      Reg16<E>::prod(S[j][mt], ident));
      }
      // ---- R = V - Kt S (V enters through an exact identity product) ----
      {
        FV SF[TPW][SK];  // -S as B-operand fragments
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int s = 0; s < SK; ++s) SF[j][s] = acc_frag_neg(S[j], s, E());
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int j = 0; j < TPW; ++j) R[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          const E* krow = &sm.k[b][16 * t + l16][0];
#pragma unroll
          for (int s = 0; s < SK; ++s) {
            const FV a = F::ld(krow, s, kg);
#pragma unroll
            for (int j = 0; j < TPW; ++j) R[j][t] = F::mma(a, SF[j][s], R[j][t]);
          }
#pragma unroll
          for (int j = 0; j < TPW; ++j) R[j][t] = Reg16<E>::rows(vr[j][t], ident, R[j][t]);
        }
      }
      if (i + 2 < nchunks) load_v(i + 2);  // prefetch (V registers are free)
      // ---- O^T = S^T Qt^T ----
      {
        FV SF[TPW][SK];
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int s = 0; s < SK; ++s) SF[j][s] = acc_frag(S[j], s, E());
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          const E* qrow = &sm.q[b][16 * t + l16][0];
#pragma unroll
          for (int s = 0; s < SK; ++s) {
            const FV qb = F::ld(qrow, s, kg);
#pragma unroll
            for (int j = 0; j < TPW; ++j) O[j][t] = F::mma(SF[j][s], qb, O[j][t]);
          }
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
// Host-side dispatch (bf16 inputs).
// ---------------------------------------------------------------------------
template <class Cfg>
static hipError_t launch_pipe_cfg(const PrefillArgs& a, hipStream_t stream) {
  const int groups = (a.num_units + 7) / 8;
  const int grid = groups * 8 * Cfg::NS;
  if (a.A_log)
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<Cfg, true>), dim3(grid), dim3(Cfg::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<Cfg, false>), dim3(grid), dim3(Cfg::NT), 0, stream, a);
  return hipGetLastError();
}

template <int GG>
static hipError_t launch_pipe_dims(int Dk, int Dv, int VS, const PrefillArgs& a, hipStream_t s) {
#define KDA_CASE(DK_, DV_, VS_) \
  if (Dk == DK_ && Dv == DV_ && VS == VS_) return launch_pipe_cfg<PrefillCfg<DK_, DV_, VS_, bf16, GG>>(a, s);
  KDA_CASE(64, 64, 64)
  KDA_CASE(64, 64, 32)
  KDA_CASE(64, 128, 128)
  KDA_CASE(64, 128, 64)
  KDA_CASE(64, 128, 32)
  KDA_CASE(128, 64, 64)
  KDA_CASE(128, 64, 32)
  KDA_CASE(128, 128, 64)
  KDA_CASE(128, 128, 32)
#undef KDA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_pipe(int Dk, int Dv, int g_group, int VS, const PrefillArgs& a, hipStream_t stream) {
  return g_group == 1 ? launch_pipe_dims<1>(Dk, Dv, VS, a, stream) : launch_pipe_dims<64>(Dk, Dv, VS, a, stream);
}

}  // namespace kda
