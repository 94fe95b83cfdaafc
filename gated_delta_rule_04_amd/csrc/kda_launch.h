// Internal interface between the C-ABI layer (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kda_common.h"

namespace kda {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* h0;
  void* o;
  float* ht;
  const int* cu_seqlens;  // NULL: batch mode
  const int* order;       // varlen: documents by decreasing length (or NULL)
  int num_units;          // N * H
  int H;
  int T;                  // batch mode: tokens per sequence; varlen: total tokens
  // Optional (bf16 path): the state entering every 64-token chunk, rounded
  // to the operand type, row-major [slot][H][Dk][Dv]; chunk c of the sequence
  // with first token t0 and index n uses slot (t0 / 64) + n + c.  NULL: not kept.
  void* hs = nullptr;
  // Optional: the fused gate and normalisation prologue.  When
  // A_log is set, q and k are raw (L2-normalised per token in the kernel),
  // g holds the gate logits f (g = -exp(A_log) softplus(f + dt_bias)) and
  // beta the logits b (beta = sigmoid(b)); A_log, dt_bias: [H][Dk / g_group].
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
};

// Backward pass (bf16): inputs, gradients and the per-chunk workspaces.
// Bytes per (slot, head) of the front tiles handed from the backward's prep
// kernel to its local kernel: X, T and P^T, the 10 lower 16x16 blocks of each
// (a 64-token chunk), bf16.
constexpr size_t kFrontTileBytes = 3 * 10 * 256 * 2;

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* g;
  const bf16* beta;
  const bf16* dout;
  const float* dht;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  bf16* dg;
  bf16* dbeta;
  float* dh0;
  const int* cu_seqlens;
  const int* order;
  const bf16* hs;   // [slot][H][DK][DV]: state entering each chunk
  bf16* fw;         // [slot][H]: -M^T as MFMA A-operand fragments (DK x DK), F = Diag(gam) - M
  float* gw;        // [slot][H][DK]: gam = e^{G_C} of each chunk
  bf16* bw;         // [slot][H]: b in accumulator tiles (DK x DV)
  bf16* dh;         // [slot][H][DK][DV]: cotangent of the state leaving each chunk
  bf16* tw;         // [slot][H]: the chunk front's X, T and P^T blocks (16x16, accumulator lane
                    // order), written by the prep kernel and read by the local kernel
  int N, H, T, slots;
};

hipError_t launch_chunk_bwd(int Dk, int Dv, int g_group, const BwdArgs& a, hipStream_t stream);

// Backward of the gate and normalisation prologue (bf16 rows [ntok][H][...]).
struct PrologueBwdArgs {
  const bf16 *q_raw, *k_raw, *f, *b_raw;  // the prologue's inputs
  const float *A_log, *dt_bias;          // [H][Dk / g_group]
  bf16 *q, *k, *g, *beta;                // prepared inputs (written by the prepare kernel)
  const bf16 *dq, *dk, *dg, *dbeta;      // their gradients (from the chunked backward)
  bf16 *dq_raw, *dk_raw, *df, *db_raw;   // gradients of the prologue's inputs
  float *part_a, *part_b;                // [blocks][H][Dk / g_group] partial sums
  float *dA_log, *ddt_bias;              // [H][Dk / g_group]
  long long ntok;                        // B * T
  int H;
};
long long prologue_bwd_blocks(long long ntok);
hipError_t launch_prologue_prepare(int Dk, int g_group, const PrologueBwdArgs& a, hipStream_t stream);
hipError_t launch_prologue_grad(int Dk, int g_group, const PrologueBwdArgs& a, hipStream_t stream);
hipError_t launch_decode(bool bf16_io, int Dk, int Dv, int g_group, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* state, void* o, int NH, hipStream_t stream);
hipError_t launch_decode_prologue(bool bf16_io, int Dk, int Dv, int g_group, const void* q, const void* k,
                                  const void* v, const void* g, const void* beta, float* state, void* o, int N, int H,
                                  const float* A_log, const float* dt_bias, hipStream_t stream);
// state_kind: 0 fp32, 1 bf16, 2 fp16 pool; o_gate NULL or the output gate's logits [N, H, Dv];
// A_log NULL for prepared inputs, else the prologue's gate parameters (raw q, k, f, b)
hipError_t launch_decode_pool(bool bf16_io, int state_kind, int Dk, int Dv, int g_group, const void* q,
                              const void* k, const void* v, const void* g, const void* beta, void* pool,
                              const int* slots, int num_slots, int H, void* o, const void* o_gate, int NH,
                              const float* A_log, const float* dt_bias, hipStream_t stream);
hipError_t launch_short_conv_fwd(bool bf16_io, const void* x, const void* weight, const void* conv0, void* y,
                                 void* conv_final, const int* cu, int num_seqs, int B, int T, int C, int W,
                                 hipStream_t s);
long long short_conv_bwd_runs(long long ntok);
hipError_t launch_short_conv_bwd(bool bf16_io, const void* x, const void* weight, const void* conv0, const void* dy,
                                 const void* dfinal, void* dx, float* dweight, void* dconv0, float* part,
                                 const int* cu, int num_seqs, int B, int T, int C, int W, hipStream_t stream);
hipError_t launch_short_conv_step(bool bf16_io, const void* x, const void* weight, void* state, void* y, int N,
                                  int C, int W, hipStream_t s);
hipError_t launch_prefill(bool bf16_io, int Dk, int Dv, int g_group, int VS, const PrefillArgs& a,
                          hipStream_t stream);
hipError_t launch_prefill_pipe(bool bf16_io, int Dk, int Dv, int g_group, int VS, const PrefillArgs& a,
                               hipStream_t stream);
hipError_t launch_varlen_order(const int* cu, int N, int T, int* order, hipStream_t stream);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);
int prefill_slice_width(bool bf16_io, int Dk, int Dv, long long units, int num_cus);
bool prefill_supported(bool bf16_io, int Dk, int Dv);

}  // namespace kda
