// C-ABI entry points of libkda.so: argument validation and kernel launches.
// Every check runs on the host before the first HIP call; see include/kda.h.

#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "kda.h"
#include "kda_common.h"
#include "kda_launch.h"


namespace {

// The chunked kernels address a 64-token span of one tensor with 32-bit
// byte offsets: 64 * H * max(Dk, Dv) * 4 bytes must fit in an int.
constexpr int kMaxChunkedHeads = 65535;

bool head_dims_ok(int Dk, int Dv, int g_group) {
  const bool d_ok = (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
  const bool g_ok = (g_group == 1 || g_group == 64) && Dk % g_group == 0;
  return d_ok && g_ok;
}

// a*b*... <= limit in int64 without overflow
bool prod_fits(std::initializer_list<long long> xs, long long limit) {
  long long p = 1;
  for (long long x : xs) {
    if (x < 0) return false;
    if (x != 0 && p > limit / x) return false;
    p *= x;
  }
  return true;
}

size_t varlen_workspace(int num_seqs) { return ((size_t)num_seqs * sizeof(int) + 255) / 256 * 256; }

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: invalid or inconsistent sizes";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown element type";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head size, decay grouping or dtype combination not supported";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
  }
  return "KDA: unknown status";
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs, int varlen, kda_dtype dt) {
  (void)Dk;
  (void)Dv;
  (void)dt;
  if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return 0;
  return varlen ? varlen_workspace(num_seqs) : 0;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free prefill: the packed-document order table (one int per
// document) lives in a file-scope device array instead of a caller workspace.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device, with that device current, and
// only that address is ever passed to a kernel.
// ---------------------------------------------------------------------------
namespace {
static __device__ __align__(256) int scratch[KDA_NOALLOC_MAX_SEQS];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` for work on `stream` (the stream's device,
// or the current device for the NULL stream); nullptr if HIP fails.
int* scratch_for(hipStream_t stream) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = static_cast<int*>(p);
  }
  return g_scratch_ptr[dev];
}
}  // namespace

namespace {
kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B, int T,
                          int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace, size_t workspace_bytes,
                          void* stream, const float* A_log, const float* dt_bias, bool noalloc = false) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (B < 0 || T < 0 || H <= 0 || H > kMaxChunkedHeads || num_seqs < 0) return KDA_ERR_SHAPE;
  if (noalloc && cu_seqlens && num_seqs > KDA_NOALLOC_MAX_SEQS) return KDA_ERR_WORKSPACE;
  if (!head_dims_ok(Dk, Dv, g_group)) return KDA_ERR_UNSUPPORTED;
  const bool bf = dt == KDA_BF16;
  if (!kda::prefill_supported(bf, Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (B != 1) return KDA_ERR_SHAPE;
  } else if (num_seqs != B) {
    return KDA_ERR_SHAPE;
  }
  const int N = num_seqs;
  // element counts must fit in int64 and units in int32
  if (!prod_fits({B, T, H, Dk > Dv ? Dk : Dv}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (!prod_fits({N, H, Dk, Dv}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (!prod_fits({B, T}, INT_MAX)) return KDA_ERR_SHAPE;
  if (!prod_fits({N, H}, INT_MAX / 16)) return KDA_ERR_SHAPE;
  const bool has_tokens = (long long)B * T > 0;
  if (has_tokens && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
  const size_t need = kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, N, varlen, dt);
  if (!noalloc && need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long units = (long long)N * H;
  if (units == 0) return KDA_OK;
  if (!has_tokens && !ht) return KDA_OK;

  int* order = nullptr;
  if (varlen) {
    order = noalloc ? scratch_for(s) : static_cast<int*>(workspace);
    if (!order) return KDA_ERR_HIP;
    if (kda::launch_varlen_order(cu_seqlens, N, T, order, s) != hipSuccess) return KDA_ERR_HIP;
  }
  kda::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.h0 = h0;
  a.o = o;
  a.ht = ht;
  a.cu_seqlens = cu_seqlens;
  a.order = order;
  a.num_units = (int)units;
  a.H = H;
  a.T = T;
  a.hs = nullptr;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  const int vs = kda::prefill_slice_width(bf, Dk, Dv, units, device_cus());
  if (kda::launch_prefill(bf, Dk, Dv, g_group, vs, a, s) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B, int T,
                         int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return chunk_fwd_impl(q, k, v, g, beta, h0, o, ht, cu_seqlens, num_seqs, B, T, H, Dk, Dv, g_group, dt, workspace,
                        workspace_bytes, stream, nullptr, nullptr);
}

kda_status kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                  const void* b_raw, const float* A_log, const float* dt_bias, const float* h0,
                                  void* o, float* ht, const int* cu_seqlens, int num_seqs, int B, int T, int H,
                                  int Dk, int Dv, int g_group, kda_dtype dt, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (H > 0 && (!A_log || !dt_bias)) return KDA_ERR_NULL;
  return chunk_fwd_impl(q_raw, k_raw, v, f, b_raw, h0, o, ht, cu_seqlens, num_seqs, B, T, H, Dk, Dv, g_group, dt,
                        workspace, workspace_bytes, stream, A_log, dt_bias);
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B,
                                 int T, int H, int Dk, int Dv, int g_group, kda_dtype dt, void* stream) {
  return chunk_fwd_impl(q, k, v, g, beta, h0, o, ht, cu_seqlens, num_seqs, B, T, H, Dk, Dv, g_group, dt, nullptr, 0,
                        stream, nullptr, nullptr, /*noalloc=*/true);
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              float* state, void* o, int N, int H, int Dk, int Dv, int g_group, kda_dtype dt,
                              void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (N < 0 || H <= 0) return KDA_ERR_SHAPE;
  if (!head_dims_ok(Dk, Dv, g_group)) return KDA_ERR_UNSUPPORTED;
  if (!prod_fits({N, H}, INT_MAX)) return KDA_ERR_SHAPE;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
  if (kda::launch_decode(dt == KDA_BF16, Dk, Dv, g_group, q, k, v, g, beta, state, o, N * H,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_recurrent_step_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                       const void* b_raw, const float* A_log, const float* dt_bias, float* state,
                                       void* o, int N, int H, int Dk, int Dv, int g_group, kda_dtype dt,
                                       void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (N < 0 || H <= 0) return KDA_ERR_SHAPE;
  if (!head_dims_ok(Dk, Dv, g_group)) return KDA_ERR_UNSUPPORTED;
  if (!prod_fits({N, H}, INT_MAX)) return KDA_ERR_SHAPE;
  if (N == 0) return KDA_OK;
  if (!q_raw || !k_raw || !v || !f || !b_raw || !A_log || !dt_bias || !state || !o) return KDA_ERR_NULL;
  if (kda::launch_decode_prologue(dt == KDA_BF16, Dk, Dv, g_group, q_raw, k_raw, v, f, b_raw, state, o, N, H, A_log,
                                  dt_bias, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"

namespace {
kda_status step_pool_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const float* A_log, const float* dt_bias, void* state_pool, const int* slots,
                          int num_slots, void* o, const void* o_gate, int N, int H, int Dk, int Dv, int g_group,
                          kda_dtype dt, kda_dtype state_dt, void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (state_dt != KDA_F32 && state_dt != KDA_BF16 && state_dt != KDA_F16) return KDA_ERR_DTYPE;
  if (N < 0 || H <= 0 || num_slots < 0) return KDA_ERR_SHAPE;
  if (!head_dims_ok(Dk, Dv, g_group)) return KDA_ERR_UNSUPPORTED;
  if (!prod_fits({N, H}, INT_MAX)) return KDA_ERR_SHAPE;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !slots || !o) return KDA_ERR_NULL;
  if (num_slots > 0 && !state_pool) return KDA_ERR_NULL;
  const int state_kind = state_dt == KDA_BF16 ? 1 : (state_dt == KDA_F16 ? 2 : 0);
  if (kda::launch_decode_pool(dt == KDA_BF16, state_kind, Dk, Dv, g_group, q, k, v, g, beta, state_pool, slots,
                              num_slots, H, o, o_gate, N * H, A_log, dt_bias,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_recurrent_step_pool(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                   void* state_pool, const int* slots, int num_slots, void* o, const void* o_gate,
                                   int N, int H, int Dk, int Dv, int g_group, kda_dtype dt, kda_dtype state_dt,
                                   void* stream) {
  return step_pool_impl(q, k, v, g, beta, nullptr, nullptr, state_pool, slots, num_slots, o, o_gate, N, H, Dk, Dv,
                        g_group, dt, state_dt, stream);
}

kda_status kda_recurrent_step_pool_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                            const void* b_raw, const float* A_log, const float* dt_bias,
                                            void* state_pool, const int* slots, int num_slots, void* o,
                                            const void* o_gate, int N, int H, int Dk, int Dv, int g_group,
                                            kda_dtype dt, kda_dtype state_dt, void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (N > 0 && H > 0 && (!A_log || !dt_bias)) return KDA_ERR_NULL;
  return step_pool_impl(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, state_pool, slots, num_slots, o, o_gate, N, H,
                        Dk, Dv, g_group, dt, state_dt, stream);
}

static bool conv_dims_ok(int C, int W) { return C > 0 && C % 8 == 0 && W >= 1 && W <= 8; }
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

kda_status kda_short_conv_fwd(const void* x, const void* weight, const void* conv0, void* y, void* conv_final,
                              const int* cu_seqlens, int num_seqs, int B, int T, int C, int W, kda_dtype dt,
                              void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (B < 0 || T < 0 || num_seqs < 0 || C <= 0) return KDA_ERR_SHAPE;
  if (!conv_dims_ok(C, W)) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens) {
    if (B != 1) return KDA_ERR_SHAPE;
  } else if (num_seqs != B) {
    return KDA_ERR_SHAPE;
  }
  if (!prod_fits({B, T}, INT_MAX) || !prod_fits({B, T, C}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (!prod_fits({num_seqs, W, C}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  const bool has_tokens = (long long)B * T > 0;
  if (has_tokens && (!x || !weight || !y)) return KDA_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(conv0) || !aligned16(conv_final)) return KDA_ERR_UNSUPPORTED;
  if (!has_tokens && !(conv_final && W > 1 && num_seqs > 0)) return KDA_OK;
  if (kda::launch_short_conv_fwd(dt == KDA_BF16, x, weight, conv0, y, conv_final, cu_seqlens, num_seqs, B, T, C, W,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

size_t kda_short_conv_bwd_workspace_bytes(int B, int T, int C, int W) {
  if (B < 0 || T < 0 || !conv_dims_ok(C, W) || !prod_fits({B, T}, INT_MAX)) return 0;
  const long long runs = kda::short_conv_bwd_runs((long long)B * T);
  if (!prod_fits({runs, W, C}, LLONG_MAX / 8)) return 0;
  return ((size_t)runs * W * C * 4 + 255) / 256 * 256;
}

kda_status kda_short_conv_bwd(const void* x, const void* weight, const void* conv0, const void* dy,
                              const void* dconv_final, void* dx, float* dweight, void* dconv0,
                              const int* cu_seqlens, int num_seqs, int B, int T, int C, int W, kda_dtype dt,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (B < 0 || T < 0 || num_seqs < 0 || C <= 0) return KDA_ERR_SHAPE;
  if (!conv_dims_ok(C, W)) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens) {
    if (B != 1) return KDA_ERR_SHAPE;
  } else if (num_seqs != B) {
    return KDA_ERR_SHAPE;
  }
  if (!prod_fits({B, T}, INT_MAX) || !prod_fits({B, T, C}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (!prod_fits({num_seqs, W, C}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  const size_t need = kda_short_conv_bwd_workspace_bytes(B, T, C, W);
  const bool has_tokens = (long long)B * T > 0;
  if (!weight || !dweight) return KDA_ERR_NULL;
  if (has_tokens && (!x || !dy || !dx)) return KDA_ERR_NULL;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(conv0) || !aligned16(dconv_final) ||
      !aligned16(dconv0))
    return KDA_ERR_UNSUPPORTED;
  if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_WORKSPACE;
  if (kda::launch_short_conv_bwd(dt == KDA_BF16, x, weight, conv0, dy, dconv_final, dx, dweight, dconv0,
                                 static_cast<float*>(workspace), cu_seqlens, num_seqs, B, T, C, W,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_short_conv_step(const void* x, const void* weight, void* conv_state, void* y, int N, int C, int W,
                               kda_dtype dt, void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (N < 0 || C <= 0) return KDA_ERR_SHAPE;
  if (!conv_dims_ok(C, W)) return KDA_ERR_UNSUPPORTED;
  if (!prod_fits({N, C}, INT_MAX) || !prod_fits({N, W, C}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (N == 0) return KDA_OK;
  if (!x || !weight || !y || (W > 1 && !conv_state)) return KDA_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(conv_state)) return KDA_ERR_UNSUPPORTED;
  if (kda::launch_short_conv_step(dt == KDA_BF16, x, weight, conv_state, y, N, C, W,
                                  static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"

namespace {
struct BwdLayout {
  size_t order, hs, fw, bw, dh, gw, tw, total;
};
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
// Slots cover every 64-token chunk of every sequence: chunk c of sequence n
// (first token t0) is slot t0 / 64 + n + c, below tokens / 64 + N + 1.
bool bwd_layout(int B, int T, int H, int Dk, int Dv, int N, bool varlen, BwdLayout& L, long long& slots) {
  if (B < 0 || T < 0 || H <= 0 || N < 0) return false;
  if (!prod_fits({B, T}, INT_MAX)) return false;
  slots = (long long)B * T / 64 + N + 1;
  if (!prod_fits({slots, H, Dk, Dv}, LLONG_MAX / 16) || !prod_fits({slots, H}, INT_MAX)) return false;
  const size_t sh = (size_t)slots * H;
  L.order = varlen ? varlen_workspace(N) : 0;
  L.hs = L.order;
  L.fw = L.hs + align256(sh * Dk * Dv * 2);
  L.bw = L.fw + align256(sh * Dk * Dk * 2);
  L.dh = L.bw + align256(sh * Dk * Dv * 2);
  L.gw = L.dh + align256(sh * Dk * Dv * 2);
  L.tw = L.gw + align256(sh * Dk * 4);
  L.total = L.tw + align256(sh * kda::kFrontTileBytes);
  return true;
}
}  // namespace

extern "C" {

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs, int varlen, kda_dtype dt) {
  (void)dt;
  BwdLayout L;
  long long slots;
  if (!bwd_layout(B, T, H, Dk, Dv, num_seqs, varlen != 0, L, slots)) return 0;
  return L.total;
}

}  // extern "C"

namespace {
// kRecompute: the backward recomputes the forward's chunk states itself.
// kSaved: the workspace already holds them (written by kda_chunk_fwd_save).
// kForwardSave: the forward only (o, optional ht), keeping the chunk states.
enum class BwdMode { kRecompute, kSaved, kForwardSave };

kda_status chunk_bwd_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const float* h0, void* o, float* ht, const void* dout, const float* dht, void* dq, void* dk,
                          void* dv, void* dg, void* dbeta, float* dh0, const int* cu_seqlens, int num_seqs, int B,
                          int T, int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                          size_t workspace_bytes, void* stream, BwdMode mode) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (B < 0 || T < 0 || H <= 0 || H > kMaxChunkedHeads || num_seqs < 0) return KDA_ERR_SHAPE;
  if (!head_dims_ok(Dk, Dv, g_group)) return KDA_ERR_UNSUPPORTED;
  if (dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (B != 1) return KDA_ERR_SHAPE;
  } else if (num_seqs != B) {
    return KDA_ERR_SHAPE;
  }
  const int N = num_seqs;
  if (!prod_fits({B, T, H, Dk > Dv ? Dk : Dv}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (!prod_fits({N, H, Dk, Dv}, LLONG_MAX / 8)) return KDA_ERR_SHAPE;
  if (!prod_fits({N, H}, INT_MAX / 16)) return KDA_ERR_SHAPE;
  BwdLayout L;
  long long slots;
  if (!bwd_layout(B, T, H, Dk, Dv, N, varlen, L, slots)) return KDA_ERR_SHAPE;
  const bool has_tokens = (long long)B * T > 0;
  const bool fwd_only = mode == BwdMode::kForwardSave;
  if (has_tokens && (!q || !k || !v || !g || !beta)) return KDA_ERR_NULL;
  if (has_tokens && fwd_only && !o) return KDA_ERR_NULL;
  if (has_tokens && !fwd_only && (!dout || !dq || !dk || !dv || !dg || !dbeta)) return KDA_ERR_NULL;
  if (!workspace || workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long units = (long long)N * H;
  if (units == 0) return KDA_OK;
  char* ws = static_cast<char*>(workspace);
  int* order = nullptr;
  if (varlen) {
    order = reinterpret_cast<int*>(ws + 0);
    if (kda::launch_varlen_order(cu_seqlens, N, T, order, s) != hipSuccess) return KDA_ERR_HIP;
  }
  // 1. forward, keeping the state entering every chunk (and o, ht when asked)
  if (mode != BwdMode::kSaved && (has_tokens || (fwd_only && ht))) {
    kda::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.h0 = h0;
    a.o = fwd_only ? o : nullptr;
    a.ht = fwd_only ? ht : nullptr;
    a.cu_seqlens = cu_seqlens;
    a.order = order;
    a.num_units = (int)units;
    a.H = H;
    a.T = T;
    a.hs = ws + L.hs;
    const int vs = kda::prefill_slice_width(true, Dk, Dv, units, device_cus());
    if (kda::launch_prefill(true, Dk, Dv, g_group, vs, a, s) != hipSuccess) return KDA_ERR_HIP;
  }
  if (fwd_only) return KDA_OK;
  // 2.-4. transfer and offset per chunk, reverse state pass, local gradients
  kda::BwdArgs b;
  b.q = static_cast<const kda::bf16*>(q);
  b.k = static_cast<const kda::bf16*>(k);
  b.v = static_cast<const kda::bf16*>(v);
  b.g = static_cast<const kda::bf16*>(g);
  b.beta = static_cast<const kda::bf16*>(beta);
  b.dout = static_cast<const kda::bf16*>(dout);
  b.dht = dht;
  b.dq = static_cast<kda::bf16*>(dq);
  b.dk = static_cast<kda::bf16*>(dk);
  b.dv = static_cast<kda::bf16*>(dv);
  b.dg = static_cast<kda::bf16*>(dg);
  b.dbeta = static_cast<kda::bf16*>(dbeta);
  b.dh0 = dh0;
  b.cu_seqlens = cu_seqlens;
  b.order = order;
  b.hs = reinterpret_cast<const kda::bf16*>(ws + L.hs);
  b.fw = reinterpret_cast<kda::bf16*>(ws + L.fw);
  b.bw = reinterpret_cast<kda::bf16*>(ws + L.bw);
  b.dh = reinterpret_cast<kda::bf16*>(ws + L.dh);
  b.gw = reinterpret_cast<float*>(ws + L.gw);
  b.tw = reinterpret_cast<kda::bf16*>(ws + L.tw);
  b.N = N;
  b.H = H;
  b.T = T;
  b.slots = has_tokens ? (int)slots : 0;
  if (kda::launch_chunk_bwd(Dk, Dv, g_group, b, s) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* h0, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                         void* dg, void* dbeta, float* dh0, const int* cu_seqlens, int num_seqs, int B, int T,
                         int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(q, k, v, g, beta, h0, nullptr, nullptr, dout, dht, dq, dk, dv, dg, dbeta, dh0, cu_seqlens,
                        num_seqs, B, T, H, Dk, Dv, g_group, dt, workspace, workspace_bytes, stream,
                        BwdMode::kRecompute);
}

kda_status kda_chunk_fwd_save(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B, int T,
                              int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(q, k, v, g, beta, h0, o, ht, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, cu_seqlens, num_seqs, B, T, H, Dk, Dv, g_group, dt, workspace, workspace_bytes, stream,
                        BwdMode::kForwardSave);
}

kda_status kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const float* h0, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                               void* dg, void* dbeta, float* dh0, const int* cu_seqlens, int num_seqs, int B, int T,
                               int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(q, k, v, g, beta, h0, nullptr, nullptr, dout, dht, dq, dk, dv, dg, dbeta, dh0, cu_seqlens,
                        num_seqs, B, T, H, Dk, Dv, g_group, dt, workspace, workspace_bytes, stream, BwdMode::kSaved);
}

}  // extern "C"

namespace {
// Workspace of the prologue backward: the chunked backward's own workspace,
// then the prepared inputs, their gradients and the parameter partial sums.
struct ProBwdLayout {
  size_t q, k, g, beta, dq, dk, dg, dbeta, pa, pb, total;
};
bool pro_bwd_layout(int B, int T, int H, int Dk, int Dv, int g_group, int N, bool varlen, ProBwdLayout& P) {
  BwdLayout L;
  long long slots;
  if (!bwd_layout(B, T, H, Dk, Dv, N, varlen, L, slots)) return false;
  if (g_group <= 0 || !prod_fits({B, T, H, Dk}, LLONG_MAX / 16)) return false;
  const size_t rows = (size_t)B * T * H, ng = (size_t)(Dk / g_group);
  const size_t nblk = (size_t)kda::prologue_bwd_blocks((long long)B * T);
  size_t o = align256(L.total);
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  P.q = take(rows * Dk * 2);
  P.k = take(rows * Dk * 2);
  P.g = take(rows * ng * 2);
  P.beta = take(rows * 2);
  P.dq = take(rows * Dk * 2);
  P.dk = take(rows * Dk * 2);
  P.dg = take(rows * ng * 2);
  P.dbeta = take(rows * 2);
  P.pa = take(nblk * H * ng * 4);
  P.pb = take(nblk * H * ng * 4);
  P.total = o;
  return true;
}
}  // namespace

extern "C" {

size_t kda_chunk_bwd_prologue_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs, int varlen,
                                              int g_group, kda_dtype dt) {
  (void)dt;
  if (!head_dims_ok(Dk, Dv, g_group) || H <= 0) return 0;
  ProBwdLayout P;
  if (!pro_bwd_layout(B, T, H, Dk, Dv, g_group, num_seqs, varlen != 0, P)) return 0;
  return P.total;
}

kda_status kda_chunk_bwd_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                  const void* b_raw, const float* A_log, const float* dt_bias, const float* h0,
                                  const void* dout, const float* dht, void* dq_raw, void* dk_raw, void* dv, void* df,
                                  void* db_raw, float* dA_log, float* ddt_bias, float* dh0, const int* cu_seqlens,
                                  int num_seqs, int B, int T, int H, int Dk, int Dv, int g_group, kda_dtype dt,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
  if (B < 0 || T < 0 || H <= 0 || H > kMaxChunkedHeads || num_seqs < 0) return KDA_ERR_SHAPE;
  if (!head_dims_ok(Dk, Dv, g_group)) return KDA_ERR_UNSUPPORTED;
  if (dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (B != 1) return KDA_ERR_SHAPE;
  } else if (num_seqs != B) {
    return KDA_ERR_SHAPE;
  }
  ProBwdLayout P;
  if (!pro_bwd_layout(B, T, H, Dk, Dv, g_group, num_seqs, varlen, P)) return KDA_ERR_SHAPE;
  if (!A_log || !dt_bias || !dA_log || !ddt_bias) return KDA_ERR_NULL;
  const bool has_tokens = (long long)B * T > 0;
  if (has_tokens && (!q_raw || !k_raw || !v || !f || !b_raw || !dout || !dq_raw || !dk_raw || !dv || !df || !db_raw))
    return KDA_ERR_NULL;
  if (!aligned16(q_raw) || !aligned16(k_raw) || !aligned16(dq_raw) || !aligned16(dk_raw)) return KDA_ERR_UNSUPPORTED;
  if (g_group == 1 && (!aligned16(f) || !aligned16(df))) return KDA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < P.total) return KDA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  kda::PrologueBwdArgs a;
  a.q_raw = static_cast<const kda::bf16*>(q_raw);
  a.k_raw = static_cast<const kda::bf16*>(k_raw);
  a.f = static_cast<const kda::bf16*>(f);
  a.b_raw = static_cast<const kda::bf16*>(b_raw);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.q = reinterpret_cast<kda::bf16*>(ws + P.q);
  a.k = reinterpret_cast<kda::bf16*>(ws + P.k);
  a.g = reinterpret_cast<kda::bf16*>(ws + P.g);
  a.beta = reinterpret_cast<kda::bf16*>(ws + P.beta);
  a.dq = reinterpret_cast<const kda::bf16*>(ws + P.dq);
  a.dk = reinterpret_cast<const kda::bf16*>(ws + P.dk);
  a.dg = reinterpret_cast<const kda::bf16*>(ws + P.dg);
  a.dbeta = reinterpret_cast<const kda::bf16*>(ws + P.dbeta);
  a.dq_raw = static_cast<kda::bf16*>(dq_raw);
  a.dk_raw = static_cast<kda::bf16*>(dk_raw);
  a.df = static_cast<kda::bf16*>(df);
  a.db_raw = static_cast<kda::bf16*>(db_raw);
  a.part_a = reinterpret_cast<float*>(ws + P.pa);
  a.part_b = reinterpret_cast<float*>(ws + P.pb);
  a.dA_log = dA_log;
  a.ddt_bias = ddt_bias;
  a.ntok = (long long)B * T;
  a.H = H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // 1. the prepared inputs; 2. the chunked backward on them; 3. the prologue's chain rule
  if (kda::launch_prologue_prepare(Dk, g_group, a, s) != hipSuccess) return KDA_ERR_HIP;
  const kda_status st = chunk_bwd_impl(a.q, a.k, v, a.g, a.beta, h0, nullptr, nullptr, dout, dht, ws + P.dq,
                                       ws + P.dk, dv, ws + P.dg, ws + P.dbeta, dh0, cu_seqlens, num_seqs, B, T, H, Dk,
                                       Dv, g_group, dt, workspace, P.q, stream, BwdMode::kRecompute);
  if (st != KDA_OK) return st;
  if (kda::launch_prologue_grad(Dk, g_group, a, s) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"
