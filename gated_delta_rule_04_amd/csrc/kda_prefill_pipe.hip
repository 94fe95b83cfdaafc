// KDA chunked prefill, gfx950 (CDNA4): one fused, software-pipelined kernel
// for bf16 and fp32 inputs.
//
// The chunked parallel form of the miniKimiK3 card's Kimi Delta Attention
// bullet ("Architecture" section).  The pages state that KDA trains through a
// chunked parallel form but give no algebra; the form below is derived from
// the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t, and is exact up to rounding.  Per head and sub-block of 16
// tokens, with S the state entering the sub-block, G_r the cumulative
// log-decay from the sub-block's start to token r and M = G_end / 2 the
// midpoint of the sub-block's decay (per key channel):
//
//   gated operands  QB = Q e^{G-M},  KB = K e^{G-M},  KD = K e^{M-G},
//                   KE = K e^{G_end - G + M'}   (M': the next sub-block's M,
//                                                0 after a chunk's last one)
//   transform       N = strictly_lower(Diag(b) KB KD^T),  P = lower_incl(QB KD^T),
//                   T = (I + N)^-1 Diag(b)                        (16 x 16, MFMA)
//   state pass      with S' = Diag(e^M) S carried instead of S:
//                   R = V - KB S';  U = T R;  O = QB S' + P U;
//                   S' <- Diag(e^{G_end - M + M'}) S' + KE^T U    (MFMA)
//
// Every exponent is referenced inside one 16-token sub-block and to the
// midpoint of its decay, so QB, KB and KD lie within e^{+-D/2} of q and k,
// D the sub-block's decay: they stay in the float range while a channel's
// log-decay summed over the sub-block is above about -140, whatever the
// decay over longer spans.  Between chunks S' is S; a chunk's first
// sub-block starts with S' = Diag(e^M) S.
//
// Design for MI355X.  A workgroup owns one (sequence, head, value slice) and
// walks that sequence in chunks of CL tokens (CL / 16 sub-blocks); nothing
// goes through HBM between the steps, so q, k, v, g, beta are read once and o
// written once.  Wavefronts are specialised:
//   - producers (one per 16 key channels) gate each chunk two steps ahead of
//     the state pass and build each sub-block's T and P one step ahead;
//   - state wavefronts (one per 16 value columns of the slice, at most four)
//     keep their columns of the fp32 state in MFMA accumulators and run the
//     sub-blocks in order, at raised issue priority (they carry the
//     recurrence).
// Each pipeline iteration i has two stages between LDS-only barriers:
//
//   stage | state wavefronts              | producers
//   ------+--------------------------------+-------------------------------------
//     P   | chunk i: second half of its    | chunk i+1: T, P of every sub-block
//         |   sub-blocks                   | chunk i+2: decay sums, beta
//     Q   | chunk i+1: first half of its   | chunk i+2: QB, KB, KE, KD, factors
//         |   sub-blocks                   |
//
// QB, KB, KE, V, T, P, beta and the state factors are double-buffered in LDS
// by chunk parity; KD is read only by the transform one stage after it is
// written and has one buffer.  The producers issue every global load (q, k,
// v, g, beta) one iteration before its use, so the loads stay in flight
// across the barriers and the state wavefronts, whose only global accesses
// are the o stores, never wait on memory.  The slices of one head are placed on
// the same XCD so that their shared q/k/g reads hit that XCD's L2.
//
// Numerics: S, N and all accumulators are fp32; MFMA operands (gated q/k, T,
// P, U and a copy of S') are rounded to the input type.  U = T R is taken in
// fp32 from the bf16 T, so R is not rounded.

#include "kda_prefill_common.h"
#include "kda_launch.h"

namespace kda {

template <typename E>
struct Tile16;  // one 16 x 16 tile in accumulator form, one lane's share
template <>
struct Tile16<bf16> {
  typedef bf16x4 type;
  __device__ __forceinline__ static type pack(const f32x4& v) { return to_bf16x4(v); }
  __device__ __forceinline__ static f32x4 unpack(const type& v) {
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
};
template <>
struct Tile16<float> {
  typedef f32x4 type;
  __device__ __forceinline__ static type pack(const f32x4& v) { return v; }
  __device__ __forceinline__ static f32x4 unpack(const type& v) { return v; }
};

template <class Cfg>
struct PipeSmem {
  typedef typename Cfg::E E;
  typedef typename Tile16<E>::type TT;
  E q[2][Cfg::CL][Cfg::KP];    // QB = Q e^{G-M}          (token-major), by chunk parity
  E k[2][Cfg::CL][Cfg::KP];    // KB = K e^{G-M}          (token-major)
  E ke[2][Cfg::CL][Cfg::KEP];  // KE = K e^{G_end-G+M'}   (token-major; bf16: swizzled)
  E kd[Cfg::CL][Cfg::KP];      // KD = K e^{M-G}          (token-major), transform only
  E v[2][Cfg::CL][Cfg::VS + Cfg::PADE];  // V rows of the slice (loaded by the producers)
  TT t[2][Cfg::NSB][64];       // -T^T of each sub-block, accumulator form
  TT p[2][Cfg::NSB][64];       // P^T of each sub-block, accumulator form
  alignas(16) float beta[2][Cfg::CL];
  alignas(16) float phi[2][Cfg::NSB][Cfg::DK];  // e^{G_end - M + M'} of each sub-block
  alignas(16) float psi[2][Cfg::DK];            // e^M of the chunk's first sub-block
  alignas(16) float gsum[Cfg::NPW][Cfg::DK];    // per-wavefront log2-decay totals
  alignas(16) float nrm[Cfg::NPW][32];          // prologue: per-wavefront inverse row norms
};

// 16x16 products whose first operand comes from LDS in accumulator form
// (lane l: M[4(l/16) + i][l % 16] of the matrix whose transpose is A), as
// Reg16<E>::prod(At, B) = A * B.  bf16: the stored operand is bf16 already.
template <typename E>
struct RegLds;
template <>
struct RegLds<bf16> {
  // A * B with A^T stored in bf16 and B an fp32 accumulator tile, B split
  // into bf16 parts hi + lo (lo = B - hi, rounded): two 16x16x16 steps whose
  // sum is within about 2^-16 of A * B, so B is not rounded to bf16.
  __device__ __forceinline__ static f32x4 prod_f32(const bf16x4& At, const f32x4& B) {
    const bf16x4 hi = to_bf16x4(B);
    const f32x4 lo = B - f32x4{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};
    const s16x4 a = __builtin_bit_cast(s16x4, At);
    const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4, hi),
                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, Reg16<bf16>::cvt(lo), c, 0, 0, 0);
  }
  // A * B with A^T an fp32 accumulator tile (rounded to bf16) and B stored
  // in bf16 in accumulator form: one 16x16x16 bf16 step.
  __device__ __forceinline__ static f32x4 prod(const f32x4& At, const bf16x4& B) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Reg16<bf16>::cvt(At), __builtin_bit_cast(s16x4, B),
                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};
template <>
struct RegLds<float> {
  __device__ __forceinline__ static f32x4 prod_f32(const f32x4& At, const f32x4& B) {
    return Reg16<float>::prod(At, B);
  }
  __device__ __forceinline__ static f32x4 prod(const f32x4& At, const f32x4& B) { return Reg16<float>::prod(At, B); }
};

// OST: the state pass leaves o in LDS and the producers store it (used when
// the kernel also keeps the chunk states: the state wavefronts' o stores and
// chunk-state stores together slow their chain; either alone does not).
template <class Cfg, bool PRO, bool OST>
__global__ __launch_bounds__(Cfg::NT) void chunk_fwd_pipe_kernel(PrefillArgs args) {
  typedef typename Cfg::T T;
  typedef typename Cfg::E E;
  typedef Frag<E> F;
  typedef typename F::V FV;
  typedef Tile16<E> TL;
  constexpr int DK = Cfg::DK, DV = Cfg::DV, VS = Cfg::VS, GG = Cfg::GG, CL = Cfg::CL, KP = Cfg::KP;
  constexpr int KEP = Cfg::KEP, NSB = Cfg::NSB, HSB = NSB / 2;
  constexpr int NS = Cfg::NS, TPW = Cfg::TPW, KT = Cfg::KT, RPB = Cfg::RPB, NPW = Cfg::NPW;
  constexpr int WPB = Cfg::WPB;
  constexpr int SK = DK / F::SLAB;  // slabs over key channels

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
  // 64-token chunk c of this sequence keeps its entering state in slot hs_slot0 + c
  const int hs_slot0 = (tok0 >> 6) + seq;
  const int nchunks = (len + CL - 1) / CL;

  const T* __restrict__ gq = static_cast<const T*>(args.q);
  const T* __restrict__ gk = static_cast<const T*>(args.k);
  const T* __restrict__ gv = static_cast<const T*>(args.v);
  const T* __restrict__ gg = static_cast<const T*>(args.g);
  const T* __restrict__ gb = static_cast<const T*>(args.beta);
  T* __restrict__ go = static_cast<T*>(args.o);
  const size_t state_off = ((size_t)seq * H + h) * DK * DV;

  f32x4 ident, nident;  // 16x16 identity and its negative, accumulator form
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ident[i] = (4 * kg + i == l16) ? 1.f : 0.f;
    nident[i] = -ident[i];
  }

  // Fragments of the 16-row block blk of a token-major operand tile.
  auto ld_rows = [&](FV (&fr)[SK], const E (*tile)[KP], int blk) {
    const E* row = &tile[0][0] + opaque(l16 * KP) + 16 * blk * KP;
#pragma unroll
    for (int s = 0; s < SK; ++s) fr[s] = F::ld(row, s, kg);
  };
  auto mma_rows = [&](const FV (&a)[SK], const FV (&b)[SK]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SK; ++s) acc = F::mma(a[s], b[s], acc);
    return acc;
  };

  if (producer) {
    // ================= producer wavefronts ===================================
    // Gating map: thread = (CPT key channels, block of RPB consecutive tokens).
    constexpr int CPT = Cfg::CPT, CG = Cfg::CG, CGN = Cfg::CGN, RBW = Cfg::RBW;
    typedef typename VecN<T, CPT>::type VC;
    typedef typename Vec8<T>::type V8;
    const int cg = tid % CGN, rb = tid / CGN;
    const int ch = CPT * cg;               // first key channel of this thread
    const int rbw = lane / CGN;            // row block within the wavefront
    const int sbw = wave / WPB;            // sub-block of this wavefront's rows
    VC rq[RPB], rk[RPB], rg[GG == 1 ? RPB : 1];
    // V rows of the slice, in 8-element units spread over the producers
    constexpr int VU = CL * VS / 8, NVL = (VU + Cfg::NA - 1) / Cfg::NA;
    V8 rv[NVL];
    T rgs[GG == 1 ? 1 : RPB], rbeta;
    // Rows past the end of the sequence read as zero through the per-chunk
    // buffer bounds.
    const int rsk = H * DK * (int)sizeof(T);         // token stride of q, k (bytes)
    const int rsg = H * (DK / GG) * (int)sizeof(T);  // token stride of g
    const int rsb = H * (int)sizeof(T);              // token stride of beta
    // prologue: -exp(A_log) and dt_bias log2(e) of this thread's channels (or group)
    constexpr int NGC = PRO ? (GG == 1 ? CPT : 1) : 1;
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
    auto chunk_rows = [&](int ck) { return min(CL, len - ck * CL); };
    auto chunk_row0 = [&](int ck) { return (size_t)(tok0 + ck * CL) * H + h; };
    // bytes of a chunk's nv rows at a token stride (0 for no rows: nothing is read)
    auto span = [&](int nv, int stride, int row_bytes) { return nv > 0 ? (nv - 1) * stride + row_bytes : 0; };
    // Every prefetch is issued, in the same order, in every iteration (the
    // last chunk again past the end), and only inside the loop (an extra
    // leading iteration issues the first chunk's), so the compiler can count
    // the loads in flight and wait only for the ones a stage uses.
    auto load_gb = [&](int ck) {  // g, beta
      const int nv = chunk_rows(ck);
      const size_t row0 = chunk_row0(ck);
      const rsrc_t bg = make_rsrc(gg + row0 * (DK / GG), span(nv, rsg, (DK / GG) * (int)sizeof(T)));
      const rsrc_t bb = make_rsrc(gb + row0, span(nv, rsb, (int)sizeof(T)));
#pragma unroll
      for (int j = 0; j < RPB; ++j) {
        const int r = rb * RPB + j;
        if constexpr (GG == 1)
          rg[j] = VecN<T, CPT>::load(bg, r * rsg + ch * (int)sizeof(T));
        else
          rgs[j] = bload<T>(bg, r * rsg + (ch / GG) * (int)sizeof(T));
      }
      rbeta = bload<T>(bb, (tid % CL) * rsb);  // threads tid < CL use theirs
    };
    const int rsv = H * DV * (int)sizeof(T);         // token stride of v (bytes)
    auto load_qk = [&](int ck) {  // q, k and the slice's V rows
      const int nv = chunk_rows(ck);
      const rsrc_t bq = make_rsrc(gq + chunk_row0(ck) * DK, span(nv, rsk, DK * (int)sizeof(T)));
      const rsrc_t bk = make_rsrc(gk + chunk_row0(ck) * DK, span(nv, rsk, DK * (int)sizeof(T)));
      const rsrc_t bv = make_rsrc(gv + chunk_row0(ck) * DV + col0, span(nv, rsv, VS * (int)sizeof(T)));
#pragma unroll
      for (int j = 0; j < RPB; ++j) rq[j] = VecN<T, CPT>::load(bq, (rb * RPB + j) * rsk + ch * (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < RPB; ++j) rk[j] = VecN<T, CPT>::load(bk, (rb * RPB + j) * rsk + ch * (int)sizeof(T));
#pragma unroll
      for (int j = 0; j < NVL; ++j) {
        const int u = tid + Cfg::NA * j;
        if (VU % Cfg::NA == 0 || u < VU)
          rv[j] = Vec8<T>::load(bv, (u / (VS / 8)) * rsv + 8 * (u % (VS / 8)) * (int)sizeof(T));
      }
    };
    float G[RPB][CPT];  // cumulative log2-decay of this thread's rows (thread-local)
    float off[CPT];     // log2-decay of the rows of this wavefront before this thread's block
    float tot[CPT];     // log2-decay over this wavefront's rows

    // ---- transform of sub-block I of the chunk in buffer b: N = A_II and
    // N^T (registers only), P^T, X = (I + N)^-1; T^T = (X Diag(b))^T and P^T
    // go to LDS in accumulator form (lane order). ----
    auto diag_job = [&](int b, int I) {
      FV kb[SK], kd[SK], qb[SK];
      ld_rows(kb, sm.k[b], I);
      ld_rows(kd, sm.kd, I);
      ld_rows(qb, sm.q[b], I);
      f32x4 N = mma_rows(kb, kd);
      f32x4 Pt = mma_rows(kd, qb);  // lane: P[16I + l16][16I + 4kg + i]
      const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[b][opaque(4 * kg) + 16 * I]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * kg + i;
        N[i] = l16 < r ? N[i] * br[i] : 0.f;  // strictly lower, rows scaled
        Pt[i] = r <= l16 ? Pt[i] : 0.f;       // lower including the diagonal
      }
      // N^T by the exact product with the identity (of N rounded to the
      // operand type, which is how the inverse's products take N anyway)
      const f32x4 Nt = Reg16<E>::prod(N, ident);
      const f32x4 X = unit_lower_inverse16<E>(N, Nt, ident);
      // -T^T in accumulator form: lane holds -T[l16][4kg + i] = -X[l16][4kg + i] b_{4kg + i}
      // (stored negated: the state pass forms -R)
      const f32x4 Tt = Reg16<E>::prod(X, ident) * (-br);
      sm.t[b][I][lane] = TL::pack(Tt);
      sm.p[b][I][lane] = TL::pack(Pt);
    };

    const int last = max(nchunks - 1, 0);

    for (int i = -3; i < nchunks; ++i) {
      const int cT = i + 1, cG = i + 2;  // chunks under transform and gating
      const int bT = cT & 1, bG = cG & 1;
      lds_barrier();  // ---------------------------------------------------- P
      if (cT >= 0 && cT < nchunks) {
        static_switch<NPW>(wave, [&](auto Wc) {
          constexpr int W = decltype(Wc)::value;
          if constexpr (W < NSB) diag_job(bT, W);
        });
      }
      if (cG >= 0 && cG < nchunks) {
        // thread-local cumulative decay; prefix over this wavefront's blocks
        float acc[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
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
            for (int c = 0; c < CPT; ++c) {
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
        if (!PRO || nvG == CL)
          gate_rows(IC<1>{});
        else
          gate_rows(IC<0>{});
        if constexpr (RBW == 1) {  // the wavefront's rows are this thread's
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            off[c] = 0.f;
            tot[c] = acc[c];
          }
        } else {  // the two row blocks are the wavefront's halves
#pragma unroll
          for (int c = 0; c < CPT; ++c) rows2_scan(acc[c], rbw, off[c], tot[c]);
        }
        if (rbw == RBW - 1) {  // this wavefront's total, for the other wavefronts
#pragma unroll
          for (int c4 = 0; c4 < CPT; c4 += CG) {
            float t4[CG];
#pragma unroll
            for (int c = 0; c < CG; ++c) t4[c] = tot[c4 + c];
            store_run<float, CG>(&sm.gsum[wave][ch + c4], t4);
          }
        }
        if (tid < CL) sm.beta[bG][tid] = PRO ? (tid < nvG ? sigmoid_f(to_f32(rbeta)) : 0.f) : to_f32(rbeta);
      }
      load_gb(min(cG + 1, last));  // prefetch (g, beta registers are free)
      lds_barrier();  // ---------------------------------------------------- Q
      if (OST && i >= 0) {
        // o of chunk i: the state pass left each sub-block's output in the
        // V rows it had read (buffer i & 1); each thread stores the units it
        // stages V into below, as whole rows of the slice, before it
        // overwrites them with chunk i + 2's V.  Without o the descriptor
        // has size zero and drops the stores.
        const int nv = chunk_rows(i);
        const rsrc_t bo = make_rsrc(go ? go + chunk_row0(i) * DV + col0 : go,
                                    go ? span(nv, rsv, VS * (int)sizeof(T)) : 0);
#pragma unroll
        for (int j = 0; j < NVL; ++j) {
          const int u = tid + Cfg::NA * j;
          if (VU % Cfg::NA == 0 || u < VU) {
            const E* src = &sm.v[i & 1][u / (VS / 8)][8 * (u % (VS / 8))];
            const int off = (u / (VS / 8)) * rsv + 8 * (u % (VS / 8)) * (int)sizeof(T);
            if constexpr (sizeof(E) == 2) {
              const u32x2 a = *reinterpret_cast<const u32x2*>(src), b = *reinterpret_cast<const u32x2*>(src + 4);
              __builtin_amdgcn_raw_buffer_store_b128(u32x4{a[0], a[1], b[0], b[1]}, bo, off, 0, 0);
            } else {
              const f32x2 a = *reinterpret_cast<const f32x2*>(src), b = *reinterpret_cast<const f32x2*>(src + 2);
              const f32x2 c = *reinterpret_cast<const f32x2*>(src + 4), d = *reinterpret_cast<const f32x2*>(src + 6);
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{a[0], a[1], b[0], b[1]}), bo, off, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{c[0], c[1], d[0], d[1]}), bo, off + 16, 0, 0);
            }
          }
        }
      }
      if (cG >= 0 && cG < nchunks) {
        // decay before this wavefront's rows within the sub-block, the
        // sub-block's total and the next sub-block's total (log2 units), from
        // the wavefronts' totals.  The position P of this wavefront in its
        // sub-block is a compile-time index, so each sum is a fixed sequence
        // of adds; the totals are added in wavefront order (this
        // wavefront's own in its place), so every wavefront of a sub-block
        // computes the same bits for its reference.
        typedef float fcg __attribute__((ext_vector_type(CG)));
        float pre[CPT], gend[CPT], gnext[CPT];
        static_switch<WPB>(wave % WPB, [&](auto Pc) {
          constexpr int P = decltype(Pc)::value;
          const int w0 = sbw * WPB;
#pragma unroll
          for (int c4 = 0; c4 < CPT; c4 += CG) {
            fcg sum = -0.f;  // x + (-0) is x: folds away
#pragma unroll
            for (int u = 0; u < WPB; ++u) {
              fcg a;
              if (u == P) {
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                  a[c] = tot[c4 + c];
                  pre[c4 + c] = sum[c];
                }
              } else {
                a = *reinterpret_cast<const fcg*>(&sm.gsum[w0 + u][ch + c4]);
              }
              sum = u == 0 ? a : sum + a;
            }
#pragma unroll
            for (int c = 0; c < CG; ++c) gend[c4 + c] = sum[c];
          }
        });
        if (sbw + 1 < NSB) {  // uniform
#pragma unroll
          for (int c4 = 0; c4 < CPT; c4 += CG) {
            fcg sum = *reinterpret_cast<const fcg*>(&sm.gsum[(sbw + 1) * WPB][ch + c4]);
#pragma unroll
            for (int u = 1; u < WPB; ++u) sum += *reinterpret_cast<const fcg*>(&sm.gsum[(sbw + 1) * WPB + u][ch + c4]);
#pragma unroll
            for (int c = 0; c < CG; ++c) gnext[c4 + c] = sum[c];
          }
        } else {
#pragma unroll
          for (int c = 0; c < CPT; ++c) gnext[c] = 0.f;
        }
        // prologue: inverse L2 norms of this thread's q and k rows (a row's
        // channels are spread over CGN consecutive lanes)
        float iq[RPB], ik[RPB];
#pragma unroll
        for (int j = 0; j < RPB; ++j) iq[j] = ik[j] = 1.f;
        if constexpr (PRO) {
          // A row spans the wavefront (CGN = 64) or its half (32), and the
          // 8 rows of that span are every lane's: the 16 sums of squares
          // (q, k) are reduced together, halving the values a lane holds at
          // each exchange (lanes l and l ^ 32 for a whole-wavefront row,
          // then l ^ 16), then summed over the 16-lane rows.  Lane 16R then
          // holds NR consecutive sums and hands their inverse roots to its
          // span through LDS (the wavefront's own slot: its LDS accesses
          // complete in order).
          constexpr int NV0 = 2 * RPB;                    // sums per lane: 16, or 8 in fp32 at d_k = 128
          constexpr int NV1 = CGN == 64 ? NV0 / 2 : NV0;  // after the exchange across halves
          constexpr int NR = NV1 / 2;                     // after the exchange across 16-lane rows
          static_assert(NV0 == 8 || NV0 == 16, "sums per row span");
          float x[NV0];
#pragma unroll
          for (int j = 0; j < RPB; ++j) {
            x[j] = sumsq(rq[j]);
            x[RPB + j] = sumsq(rk[j]);
          }
          auto swap_add = [](float a, float b, bool by32) {
            const unsigned ab = __builtin_bit_cast(unsigned, a), bb = __builtin_bit_cast(unsigned, b);
            const auto r = by32 ? __builtin_amdgcn_permlane32_swap(ab, bb, false, false)
                                : __builtin_amdgcn_permlane16_swap(ab, bb, false, false);
            return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
          };
          if constexpr (CGN == 64) {
#pragma unroll
            for (int p = 0; p < NV1; ++p) x[p] = swap_add(x[p], x[p + NV1], true);  // sum p + NV1 (lane >= 32)
          }
#pragma unroll
          for (int p = 0; p < NR; ++p) x[p] = swap_add(x[p], x[p + NR], false);  // sum p + NR ((lane / 16) % 2)
          float r8[NR];
#pragma unroll
          for (int p = 0; p < NR; ++p) r8[p] = __builtin_amdgcn_rsqf(row_sum<16>(x[p]) + kNormEps);
          // the span's NV0 results in its slot: lane 16R writes sums
          // NR R .. NR R + NR - 1 (CGN = 64), or NR (R % 2) .. of its half (CGN = 32)
          float* slot = &sm.nrm[wave][CGN == 64 ? 0 : NV0 * (kg >> 1)];
          if (l16 == 0) {
            float* dst = slot + NR * (CGN == 64 ? kg : (kg & 1));
            if constexpr (NR == 2) {
              *reinterpret_cast<f32x2*>(dst) = f32x2{r8[0], r8[1]};
            } else {
#pragma unroll
              for (int p = 0; p < NR; p += 4)
                *reinterpret_cast<f32x4*>(dst + p) = f32x4{r8[p], r8[p + 1], r8[p + 2], r8[p + 3]};
            }
          }
          __builtin_amdgcn_wave_barrier();
          asm volatile("" ::: "memory");
#pragma unroll
          for (int j = 0; j < RPB; j += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(slot + j);
            const f32x4 b = *reinterpret_cast<const f32x4*>(slot + RPB + j);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              iq[j + i] = a[i];
              ik[j + i] = b[i];
            }
          }
        }
        // CG channels at a time: the references M of this sub-block and M'
        // of the next one in the chunk (0 after the chunk's last sub-block);
        // KE = KD e^{G_end - M} e^{M'} (two factors that each stay in range
        // inside the decay domain; a product that underflows there is below
        // e^-87 of what it is added to); the sub-block's state factor
        // e^{G_end - M + M'}; then the gated operands QB, KB, KE, KD
        // (token-major) of this thread's rows.
        const bool writer = wave % WPB == 0 && rbw == 0;  // one per (sub-block, channel group)
#pragma unroll
        for (int c4 = 0; c4 < CPT; c4 += CG) {
          // base: the decay before this thread's rows, less M; fe1 = e^{G_end - M} = e^M
          float base[CG], fe1[CG], fe2[CG];
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const float mid = 0.5f * gend[c4 + c];
            base[c] = pre[c4 + c] + off[c4 + c] - mid;
            fe1[c] = fast_exp2(mid);
            fe2[c] = fast_exp2(0.5f * gnext[c4 + c]);
          }
#pragma unroll
          for (int j = 0; j < RPB; ++j) {
            const int r = rb * RPB + j;
            float qo[CG], ko[CG], eo[CG], dd[CG];
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const float x = base[c] + G[j][c4 + c];  // G - M at this row
              const float el = fast_exp2(x), er = fast_exp2(-x);
              const float kx = elem(rk[j], c4 + c) * ik[j];
              qo[c] = elem(rq[j], c4 + c) * iq[j] * el;
              ko[c] = kx * el;
              dd[c] = kx * er;
              eo[c] = (dd[c] * fe1[c]) * fe2[c];
            }
            const int cc = ch + c4;
            store_run<E, CG>(&sm.q[bG][r][cc], qo);
            store_run<E, CG>(&sm.k[bG][r][cc], ko);
            store_run<E, CG>(&sm.kd[r][cc], dd);
            if constexpr (Cfg::TR)
              store_run<E, CG>(&sm.ke[bG][r][4 * ((cc >> 2) ^ kh_swizzle(r)) + (cc & 3)], eo);
            else
              store_run<E, CG>(&sm.ke[bG][r][cc], eo);
          }
          if (writer) {  // the state factors of the sub-block (and e^M of a chunk's first)
            float ph[CG];
#pragma unroll
            for (int c = 0; c < CG; ++c) ph[c] = fe1[c] * fe2[c];
            store_run<float, CG>(&sm.phi[bG][sbw][ch + c4], ph);
            if (sbw == 0) store_run<float, CG>(&sm.psi[bG][ch + c4], fe1);
          }
        }
#pragma unroll
        for (int j = 0; j < NVL; ++j) {
          const int u = tid + Cfg::NA * j;
          if (VU % Cfg::NA == 0 || u < VU) {  // the loaded elements as they are
            E* dst = &sm.v[bG][u / (VS / 8)][8 * (u % (VS / 8))];
            if constexpr (sizeof(E) == 2) {
              *reinterpret_cast<bf16x4*>(dst) = __builtin_shufflevector(rv[j], rv[j], 0, 1, 2, 3);
              *reinterpret_cast<bf16x4*>(dst + 4) = __builtin_shufflevector(rv[j], rv[j], 4, 5, 6, 7);
            } else {
              store4<E>(dst, f32x4{elem(rv[j], 0), elem(rv[j], 1), elem(rv[j], 2), elem(rv[j], 3)});
              store4<E>(dst + 4, f32x4{elem(rv[j], 4), elem(rv[j], 5), elem(rv[j], 6), elem(rv[j], 7)});
            }
          }
        }
      }
      load_qk(min(cG + 1, last));  // prefetch (q, k, v registers are free)
    }
    return;
  }

  // ================= state wavefronts ======================================
  const int bw = wave - NPW;  // state wavefront index
  // The state pass carries the recurrence; its short VALU/LDS/MFMA bursts are
  // issued ahead of the producers' long VALU streams on the same SIMD.
  __builtin_amdgcn_s_setprio(2);
  // S' = Diag(e^M) S of the current sub-block (S itself between chunks):
  // rows (key channels) 16mt + 4kg + i, column l16
  f32x4 S[TPW][KT];
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

  const int rsv = H * DV * (int)sizeof(T);  // token stride of o (bytes)
  typedef typename Row4<T>::type VR;

  // One sub-block t of the chunk ck in buffer b.
  auto sub_step = [&](int b, int ck, int t) {
    // operands of the sub-block from LDS first: none depends on the state
    FV ka[SK], qa[SK];
    {
      const E* krow = &sm.k[b][0][0] + opaque(l16 * KP) + 16 * t * KP;
      const E* qrow = &sm.q[b][0][0] + opaque(l16 * KP) + 16 * t * KP;
#pragma unroll
      for (int s = 0; s < SK; ++s) {
        ka[s] = F::ld(krow, s, kg);
        qa[s] = F::ld(qrow, s, kg);
      }
    }
    VR vr[TPW];  // lane: 4 columns of token 16t + l16
#pragma unroll
    for (int j = 0; j < TPW; ++j)
      vr[j] = *reinterpret_cast<const VR*>(&sm.v[b][16 * t + l16][16 * (TPW * bw + j) + 4 * kg]);
    const auto Tt = sm.t[b][t][lane];
    const auto Pt = sm.p[b][t][lane];
    FV SF[TPW][SK];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int s = 0; s < SK; ++s) SF[j][s] = acc_frag(S[j], s, E());
    // ---- -R = KB S - V (V enters through an exact product with the negated
    // identity; the transform is stored negated, so that U = (-T)(-R)) ----
    f32x4 R[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) R[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SK; ++s)
#pragma unroll
      for (int j = 0; j < TPW; ++j) R[j] = F::mma(ka[s], SF[j][s], R[j]);
#pragma unroll
    for (int j = 0; j < TPW; ++j) R[j] = Reg16<E>::rows(vr[j], nident, R[j]);
    // ---- O^T = S^T QB^T ----
    f32x4 O[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SK; ++s)
#pragma unroll
      for (int j = 0; j < TPW; ++j) O[j] = F::mma(SF[j][s], qa[s], O[j]);
    // ---- U = (-T)(-R) (-R unrounded), O^T += U^T P^T, write o of the sub-block ----
    f32x4 U[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      U[j] = RegLds<E>::prod_f32(Tt, R[j]);
      O[j] += RegLds<E>::prod(U[j], Pt);
    }
    if constexpr (OST) {
      // o of the sub-block into the V elements this lane read above (no
      // other wavefront reads them); the producers store the chunk's o to
      // HBM as whole rows one stage later
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        store4<E>(&sm.v[b][16 * t + l16][16 * (TPW * bw + j) + 4 * kg], O[j]);
    } else {  // no branch: without o the descriptor has size zero and drops the stores
      const int nv = min(CL, len - ck * CL) - 16 * t;
      const bool live = go != nullptr && nv > 0;
      const rsrc_t bo = make_rsrc(live ? go + ((size_t)(tok0 + ck * CL + 16 * t) * H + h) * DV + col0 : go,
                                  live ? (nv - 1) * rsv + VS * (int)sizeof(T) : 0);
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        bstore4(O[j], bo, l16 * rsv + (16 * (TPW * bw + j) + 4 * kg) * (int)sizeof(T), T());
    }
    // ---- S' <- Diag(e^{G_end - M + M'}) S' + KE^T U ----
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.phi[b][t][16 * mt + 4 * kg]);
#pragma unroll
      for (int j = 0; j < TPW; ++j) S[j][mt] *= gm;
      if constexpr (Cfg::TR) {
        // (KE^T) rows 16mt .. 16mt+15 over the sub-block's 16 tokens: in each
        // 16-lane group a transposing read hands lane l16 element l16 % 4 of
        // the 4-element pieces addressed by lanes l16 / 4 + {0, 4, 8, 12}, so
        // lane 4e + q of group kg addresses token 16t + 4kg + e, channels
        // 16mt + 4q .. 16mt + 4q + 3 (units XOR-permuted by token / 4).
        const int e = l16 >> 2, q = l16 & 3;
        const bf16* p = &sm.ke[b][0][0] + (16 * t + 4 * kg + e) * KEP + 4 * (4 * mt + (q ^ kg));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          S[j][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, Reg16<bf16>::cvt(U[j]), S[j][mt], 0, 0, 0);
      } else {
        // fp32: step s takes tokens 4kg + s of the sub-block (element s of U's tile)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float a = sm.ke[b][16 * t + 4 * kg + s][16 * mt + l16];
#pragma unroll
          for (int j = 0; j < TPW; ++j) S[j][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, U[j][s], S[j][mt], 0, 0, 0);
        }
      }
    }
  };

  for (int i = -3; i < nchunks; ++i) {  // the same iterations as the producers'
    lds_barrier();  // ------------------------------------------------------ P
    if (i >= 0) {
      const int b = i & 1;
#pragma unroll
      for (int t = 0; t < HSB; ++t) sub_step(b, i, HSB + t);
    }
    lds_barrier();  // ------------------------------------------------------ Q
    if (i + 1 >= 0 && i + 1 < nchunks) {
      const int c = i + 1, b = c & 1;
      // ---- optional: the state entering each 64-token chunk, in the operand
      // type, as 16x16 tiles (rows of four columns through an exact
      // transposing product; each tile one contiguous 512-byte store) ----
      if constexpr (Cfg::TR && CL == 64) {
        if (args.hs) {
          E* hs = static_cast<E*>(args.hs) + ((size_t)(hs_slot0 + c) * H + h) * DK * DV;
#pragma unroll
          for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
              store4<E>(hs + tile_off<DV>(16 * mt + l16, col0 + 16 * (TPW * bw + j) + 4 * kg),
                        Reg16<E>::prod(S[j][mt], ident));
        }
      }
      // ---- S' = Diag(e^M) S for the chunk's first sub-block ----
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        const f32x4 ps = *reinterpret_cast<const f32x4*>(&sm.psi[b][16 * mt + 4 * kg]);
#pragma unroll
        for (int j = 0; j < TPW; ++j) S[j][mt] *= ps;
      }
#pragma unroll
      for (int t = 0; t < HSB; ++t) sub_step(b, c, t);
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
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <class Cfg>
static hipError_t launch_pipe_cfg(const PrefillArgs& a, hipStream_t stream) {
  const int groups = (a.num_units + 7) / 8;
  const int grid = groups * 8 * Cfg::NS;
  // the producers store o when the chunk states are kept too (bf16, 64-token chunks)
  constexpr bool keeps = Cfg::TR && Cfg::CL == 64;
  if (keeps && a.hs && a.o) {
    if (a.A_log)
      hipLaunchKernelGGL((chunk_fwd_pipe_kernel<Cfg, true, keeps>), dim3(grid), dim3(Cfg::NT), 0, stream, a);
    else
      hipLaunchKernelGGL((chunk_fwd_pipe_kernel<Cfg, false, keeps>), dim3(grid), dim3(Cfg::NT), 0, stream, a);
  } else if (a.A_log) {
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<Cfg, true, false>), dim3(grid), dim3(Cfg::NT), 0, stream, a);
  } else {
    hipLaunchKernelGGL((chunk_fwd_pipe_kernel<Cfg, false, false>), dim3(grid), dim3(Cfg::NT), 0, stream, a);
  }
  return hipGetLastError();
}

template <int GG>
static hipError_t launch_pipe_bf16(int Dk, int Dv, int VS, const PrefillArgs& a, hipStream_t s) {
#define KDA_CASE(DK_, DV_, VS_) \
  if (Dk == DK_ && Dv == DV_ && VS == VS_) return launch_pipe_cfg<PrefillCfg<DK_, DV_, VS_, bf16, GG, 64>>(a, s);
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

// fp32: 64-token chunks at 64 key channels, 32-token chunks at 128 (the
// double-buffered fp32 operand tiles must fit the 160 KB of LDS).
template <int GG>
static hipError_t launch_pipe_f32(int Dk, int Dv, int VS, const PrefillArgs& a, hipStream_t s) {
#define KDA_CASE(DK_, DV_, VS_, CL_) \
  if (Dk == DK_ && Dv == DV_ && VS == VS_) return launch_pipe_cfg<PrefillCfg<DK_, DV_, VS_, float, GG, CL_>>(a, s);
  KDA_CASE(64, 64, 32, 64)
  KDA_CASE(64, 64, 16, 64)
  KDA_CASE(64, 128, 32, 64)
  KDA_CASE(64, 128, 16, 64)
  KDA_CASE(128, 64, 32, 32)
  KDA_CASE(128, 64, 16, 32)
  KDA_CASE(128, 128, 32, 32)
  KDA_CASE(128, 128, 16, 32)
#undef KDA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_pipe(bool bf16_io, int Dk, int Dv, int g_group, int VS, const PrefillArgs& a,
                               hipStream_t stream) {
  if (bf16_io)
    return g_group == 1 ? launch_pipe_bf16<1>(Dk, Dv, VS, a, stream) : launch_pipe_bf16<64>(Dk, Dv, VS, a, stream);
  return g_group == 1 ? launch_pipe_f32<1>(Dk, Dv, VS, a, stream) : launch_pipe_f32<64>(Dk, Dv, VS, a, stream);
}

}  // namespace kda
