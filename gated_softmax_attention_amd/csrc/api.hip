// libgsa C ABI: argument validation, device checks, dispatch to the gfx950 kernels.
// The declarations and their contracts are in include/gsa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <initializer_list>
#include <string>

#include "gsa.h"

namespace gsa {
hipError_t launch_gate_gemm(const void* X, const void* W, float* G, int64_t M, int64_t K, int64_t N,
                            bool bf16_inputs, int act, hipStream_t stream);
hipError_t launch_attn_fwd(const void* Q, const void* K, const void* V, const float* G, void* Y,
                           float* Lse, int B, int S, int Skv, int Hq, int Hkv, int D, int mode,
                           bool bf16_inputs, hipStream_t stream);
hipError_t launch_decode_bf16(const void* Q, const void* K, const void* V, const float* G, void* Y,
                              void* workspace, int B, int L, int Hq, int Hkv, int D, int mode,
                              int nsplit, hipStream_t stream);
int64_t decode_auto_splits(int64_t B, int64_t L, int64_t Hq, int64_t Hkv);
int64_t decode_chunk(int64_t L, int64_t nsplit);
hipError_t launch_attn_bwd(const void* Q, const void* K, const void* V, const void* dYg, const void* Yg,
                           const float* G, const float* Lse, void* dQ, void* dK, void* dV, void* dY,
                           float* Stat, void* dZ, float* part, int B, int S, int Hq, int Hkv, int D,
                           int mode, hipStream_t stream, hipStream_t dq_stream, hipEvent_t fork);
int bwd_kv_slices(int B, int S, int Hq, int Hkv, int D);
hipError_t launch_decode_variant_bf16(const void* Q, const void* K, const void* V, const float* G, void* Y,
                                      void* workspace, int B, int L, int Hq, int Hkv, int D, int layout, int add,
                                      int rms, int nsplit, hipStream_t st);
hipError_t launch_attn_fwd_variant_f32_decode(const void* Q, const void* K, const void* V, const float* G,
                                              void* Y, int B, int L, int Hq, int Hkv, int D, int layout, int add,
                                              int rms, hipStream_t stream);
hipError_t launch_project_qkvg(const void* X, const void* W, void* Q, void* Kp, void* V, float* G, int64_t M,
                               int64_t K, int64_t nq, int64_t nkv, int64_t ng, hipStream_t stream);
hipError_t launch_attn_fwd_variant(const void* Q, const void* K, const void* V, const float* G, void* Y,
                                   float* Lse, int B, int S, int Hq, int Hkv, int D, int layout, int add,
                                   int rms, bool bf16_inputs, hipStream_t stream);
hipError_t launch_value_gate(const void* V, const float* G, void* Vout, int64_t rows, int Hkv, int D,
                             bool headwise, bool bf16_inputs, hipStream_t st);
hipError_t launch_first_token_share(const void* Q, const void* K, const float* Lse, float* F, float* head_mean,
                                    int B, int S, int Hq, int Hkv, int D, bool bf16_inputs, hipStream_t st);
size_t gate_splitk_workspace_bytes(int64_t M, int64_t K, int64_t N);
int64_t gate_splitk_splits(int64_t M, int64_t K, int64_t N);
hipError_t launch_gate_gemm_splitk_parts(const void* X, const void* W, float* part, int64_t M, int64_t K, int64_t N,
                                         hipStream_t stream);
hipError_t launch_decode_gateparts_bf16(const void* Q, const void* K, const void* V, const float* gate_part,
                                        int gsplits, void* Y, void* workspace, int B, int L, int Hq, int Hkv, int D,
                                        int nsplit, hipStream_t st);
hipError_t launch_gate_gemm_splitk(const void* X, const void* W, float* G, float* part, int64_t M, int64_t K,
                                   int64_t N, int act, hipStream_t stream);
hipError_t launch_attn_fwd_value_gated(const void* Q, const void* K, const void* V, const float* Gv, void* Y,
                                       float* Lse, int B, int S, int Hq, int Hkv, int D, bool headwise,
                                       bool bf16_inputs, hipStream_t stream);
hipError_t launch_gate_head_mean(const float* G, float* Gs, int64_t M, int Hq, int D, hipStream_t st);
int bwd_stat_rows(int S);
hipError_t launch_bwd_gemm_dx(const void* dZ, const void* W, void* dX, int64_t M, int64_t d_model,
                              int64_t N, hipStream_t st);
hipError_t launch_bwd_gemm_dw(const void* X, const void* dZ, float* dW, float* partials, int64_t M,
                              int64_t d_model, int64_t N, int64_t splits, hipStream_t st);
int64_t bwd_dw_splits(int64_t M, int64_t d_model, int64_t N);
}  // namespace gsa

namespace {

thread_local std::string g_last_error;

gsa_status fail(gsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gsa_status ok() {
  g_last_error.clear();
  return GSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kIntMax = 0x7fffffff;

// The product of non-negative sizes is at most lim, computed without
// overflowing (a product that does not fit int64 is not at most lim).  Every
// size check multiplies through this, so arbitrary int64 arguments cannot make
// the checks themselves overflow.
bool prod_le(std::initializer_list<int64_t> xs, int64_t lim) {
  int64_t p = 1;
  for (int64_t x : xs) {
    if (x < 0 || __builtin_mul_overflow(p, x, &p)) return false;
  }
  return p <= lim;
}
constexpr int64_t kElemMax = (int64_t)1 << 40;   // no tensor of more elements fits a GPU

// Per-device check that the device is a gfx950 part, done once per device.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];  // 1 = gfx950, 0 = other
char g_dev_arch[kMaxDevices][64];

gsa_status check_device() {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(GSA_ERR_NO_DEVICE, "no HIP device is visible");
  }
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(GSA_ERR_NO_DEVICE, "hipGetDevice failed");
  }
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      snprintf(g_dev_arch[dev], sizeof g_dev_arch[dev], "%s", prop.gcnArchName);
      g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    } else {
      (void)hipGetLastError();
      snprintf(g_dev_arch[dev], sizeof g_dev_arch[dev], "unknown");
      g_dev_ok[dev] = 0;
    }
  });
  if (!g_dev_ok[dev])
    return fail(GSA_ERR_UNSUPPORTED, "device %d is %s; libgsa is built for gfx950 only", dev,
                g_dev_arch[dev]);
  return GSA_OK;
}

gsa_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

gsa_status check_dtype(const char* fn, int dtype) {
  if (dtype != GSA_FP32 && dtype != GSA_BF16)
    return fail(GSA_ERR_UNSUPPORTED, "%s: dtype %d is not GSA_FP32 or GSA_BF16", fn, dtype);
  return GSA_OK;
}

// S is the key/value length; Sq the query rows per batch (S for prefill, 1 for decode).
gsa_status check_attn_shape(const char* fn, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                            int mode, const float* G, int64_t Sq = -1) {
  if (Sq < 0) Sq = S;
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0)
    return fail(GSA_ERR_INVALID_ARG, "%s: sizes must be positive (B=%lld S=%lld Hq=%lld Hkv=%lld D=%lld)",
                fn, (long long)B, (long long)S, (long long)Hq, (long long)Hkv, (long long)D);
  if (Hq % Hkv != 0)
    return fail(GSA_ERR_INVALID_ARG, "%s: Hq=%lld is not a multiple of Hkv=%lld", fn, (long long)Hq,
                (long long)Hkv);
  if (mode != GSA_GATE_NONE && mode != GSA_GATE_ELEMENTWISE && mode != GSA_GATE_HEADWISE)
    return fail(GSA_ERR_INVALID_ARG, "%s: unknown gate mode %d", fn, mode);
  if ((mode == GSA_GATE_NONE) != (G == nullptr))
    return fail(GSA_ERR_INVALID_ARG, "%s: G must be NULL exactly when mode is GSA_GATE_NONE", fn);
  if (D != 64 && D != 128)
    return fail(GSA_ERR_UNSUPPORTED, "%s: head dim %lld is not supported (64 or 128)", fn, (long long)D);
  if (!prod_le({B, S}, kIntMax) || Hq > 4096 || Hkv > 4096)
    return fail(GSA_ERR_UNSUPPORTED, "%s: sizes exceed the supported range", fn);
  // the kernels address one batch's Q / K / V rows with 32-bit byte offsets
  // (bounded here at the float32 size)
  if (!prod_le({Sq, Hq, D, 4}, kIntMax) || !prod_le({S, Hkv, D, 4}, kIntMax))
    return fail(GSA_ERR_UNSUPPORTED, "%s: one batch of Q or K/V exceeds 2 GiB", fn);
  return GSA_OK;
}

}  // namespace

extern "C" {

int gsa_version(void) { return 100; }

const char* gsa_status_string(int status) {
  switch (status) {
    case GSA_OK: return "GSA_OK";
    case GSA_ERR_INVALID_ARG: return "GSA_ERR_INVALID_ARG";
    case GSA_ERR_UNSUPPORTED: return "GSA_ERR_UNSUPPORTED";
    case GSA_ERR_MISALIGNED: return "GSA_ERR_MISALIGNED";
    case GSA_ERR_WORKSPACE: return "GSA_ERR_WORKSPACE";
    case GSA_ERR_NO_DEVICE: return "GSA_ERR_NO_DEVICE";
    case GSA_ERR_HIP: return "GSA_ERR_HIP";
    default: return "GSA_ERR_UNKNOWN";
  }
}

const char* gsa_last_error_message(void) { return g_last_error.c_str(); }

gsa_status gsa_gate_logits(const void* X, const void* W, float* G, int64_t M, int64_t d_model,
                           int64_t N, int dtype, int activation, void* stream) {
  if (!X || !W || !G) return fail(GSA_ERR_INVALID_ARG, "gsa_gate_logits: null pointer");
  if (M <= 0 || d_model <= 0 || N <= 0)
    return fail(GSA_ERR_INVALID_ARG, "gsa_gate_logits: sizes must be positive (M=%lld d_model=%lld N=%lld)",
                (long long)M, (long long)d_model, (long long)N);
  if (gsa_status st = check_dtype("gsa_gate_logits", dtype)) return st;
  if (activation < GSA_ACT_IDENTITY || activation > GSA_ACT_SILU)
    return fail(GSA_ERR_INVALID_ARG, "gsa_gate_logits: activation %d is not a gsa_activation", activation);
  if (d_model % 8 != 0)
    return fail(GSA_ERR_UNSUPPORTED, "gsa_gate_logits: d_model=%lld is not a multiple of 8",
                (long long)d_model);
  if (M > kIntMax || d_model > kIntMax || N > kIntMax || !prod_le({M, d_model}, kElemMax) ||
      !prod_le({d_model, N}, kElemMax) || !prod_le({M, N}, kElemMax))
    return fail(GSA_ERR_UNSUPPORTED, "gsa_gate_logits: sizes exceed the supported range");
  if (!aligned16(X) || !aligned16(W) || !aligned16(G))
    return fail(GSA_ERR_MISALIGNED, "gsa_gate_logits: X, W and G must be 16-byte aligned");
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_gate_gemm(X, W, G, M, d_model, N, dtype == GSA_BF16, activation,
                                          (hipStream_t)stream),
                    "gsa_gate_logits launch");
}

size_t gsa_gate_logits_workspace_bytes(int64_t M, int64_t d_model, int64_t N, int dtype) {
  if (M <= 0 || d_model <= 0 || N <= 0 || dtype != GSA_BF16 || d_model % 8 != 0) return 0;
  if (M > kIntMax || d_model > kIntMax || N > kIntMax) return 0;
  return gsa::gate_splitk_workspace_bytes(M, d_model, N);
}

gsa_status gsa_gate_logits_ws(const void* X, const void* W, float* G, int64_t M, int64_t d_model, int64_t N,
                              int dtype, int activation, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gsa_gate_logits_ws";
  const size_t need = gsa_gate_logits_workspace_bytes(M, d_model, N, dtype);
  if (need == 0) {   // a shape without the split-K path: exactly gsa_gate_logits
    gsa_status st = gsa_gate_logits(X, W, G, M, d_model, N, dtype, activation, stream);
    return st;
  }
  if (!X || !W || !G) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (activation < GSA_ACT_IDENTITY || activation > GSA_ACT_SILU)
    return fail(GSA_ERR_INVALID_ARG, "%s: activation %d is not a gsa_activation", fn, activation);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(X) || !aligned16(W) || !aligned16(G) || !aligned16(workspace))
    return fail(GSA_ERR_MISALIGNED, "%s: X, W, G and the workspace must be 16-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_gate_gemm_splitk(X, W, G, (float*)workspace, M, d_model, N, activation,
                                                 (hipStream_t)stream),
                    fn);
}

}  // extern "C"

namespace {
gsa_status forward_impl(const char* fn, const void* Q, const void* K, const void* V, const float* G,
                        void* Y, float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                        int64_t D, int mode, int dtype, void* stream) {
  if (!Q || !K || !V || !Y) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (gsa_status st = check_attn_shape(fn, B, S, Hq, Hkv, D, mode, G)) return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Y) || (G && !aligned16(G)))
    return fail(GSA_ERR_MISALIGNED, "%s: Q, K, V, G and Y must be 16-byte aligned", fn);
  if (LSE && ((uintptr_t)LSE % 4) != 0)
    return fail(GSA_ERR_MISALIGNED, "%s: LSE must be 4-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_attn_fwd(Q, K, V, G, Y, LSE, (int)B, (int)S, (int)S, (int)Hq, (int)Hkv,
                                         (int)D, mode, dtype == GSA_BF16, (hipStream_t)stream),
                    fn);
}
}  // namespace

extern "C" {

gsa_status gsa_forward(const void* Q, const void* K, const void* V, const float* G, void* Y,
                       int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int mode, int dtype,
                       void* stream) {
  return forward_impl("gsa_forward", Q, K, V, G, Y, nullptr, B, S, Hq, Hkv, D, mode, dtype, stream);
}

gsa_status gsa_forward_lse(const void* Q, const void* K, const void* V, const float* G, void* Y,
                           float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                           int mode, int dtype, void* stream) {
  if (!LSE) return fail(GSA_ERR_INVALID_ARG, "gsa_forward_lse: null pointer");
  return forward_impl("gsa_forward_lse", Q, K, V, G, Y, LSE, B, S, Hq, Hkv, D, mode, dtype, stream);
}

int64_t gsa_decode_num_splits(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int num_splits) {
  if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || num_splits < 0) return 0;
  if (!prod_le({B, L}, kIntMax) || Hq > 4096 || D > 4096) return 0;   // gsa_decode's range
  int64_t ns = num_splits > 0 ? num_splits : gsa::decode_auto_splits(B, L, Hq, Hkv);
  if (ns > L) ns = L;
  // every split gets at least one key: the effective count after rounding the chunk
  const int64_t chunk = gsa::decode_chunk(L, ns);
  return (L + chunk - 1) / chunk;
}

size_t gsa_decode_workspace_bytes(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D,
                                  int num_splits) {
  const int64_t ns = gsa_decode_num_splits(B, L, Hq, Hkv, D, num_splits);
  if (ns == 0 || !prod_le({B, Hq, ns, D + 4, (int64_t)sizeof(float)}, kElemMax)) return 0;
  return (size_t)(B * Hq * ns * (D + 4)) * sizeof(float);
}

gsa_status gsa_decode(const void* Q, const void* Kc, const void* Vc, const float* G, void* Y, int64_t B,
                      int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int mode, int dtype, int num_splits,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!Q || !Kc || !Vc || !Y) return fail(GSA_ERR_INVALID_ARG, "gsa_decode: null pointer");
  if (gsa_status st = check_attn_shape("gsa_decode", B, L, Hq, Hkv, D, mode, G, 1)) return st;
  if (gsa_status st = check_dtype("gsa_decode", dtype)) return st;
  if (num_splits < 0) return fail(GSA_ERR_INVALID_ARG, "gsa_decode: num_splits must be >= 0");
  if (!prod_le({B, L}, kIntMax)) return fail(GSA_ERR_UNSUPPORTED, "gsa_decode: B*L exceeds the supported range");
  if (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(Y) || (G && !aligned16(G)))
    return fail(GSA_ERR_MISALIGNED, "gsa_decode: Q, Kc, Vc, G and Y must be 16-byte aligned");
  size_t need = 0;
  int64_t ns = 0;
  if (dtype == GSA_BF16) {
    ns = gsa_decode_num_splits(B, L, Hq, Hkv, D, num_splits);
    need = gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits);
    if (workspace_bytes < need || (need > 0 && workspace == nullptr))
      return fail(GSA_ERR_WORKSPACE, "gsa_decode: workspace of %zu bytes needed, %zu given", need,
                  workspace_bytes);
    if (workspace && !aligned16(workspace))
      return fail(GSA_ERR_MISALIGNED, "gsa_decode: workspace must be 16-byte aligned");
  }
  if (gsa_status st = check_device()) return st;
  if (dtype == GSA_BF16)
    return hip_result(gsa::launch_decode_bf16(Q, Kc, Vc, G, Y, workspace, (int)B, (int)L, (int)Hq,
                                              (int)Hkv, (int)D, mode, (int)ns, (hipStream_t)stream),
                      "gsa_decode launch");
  // float32: the general kernel with one query row aligned to the end of the cache
  return hip_result(gsa::launch_attn_fwd(Q, Kc, Vc, G, Y, nullptr, (int)B, 1, (int)L, (int)Hq, (int)Hkv, (int)D,
                                         mode, false, (hipStream_t)stream),
                    "gsa_decode launch");
}

}  // extern "C"

namespace {
// Device-resident scratch for gsa_decode_noalloc: the split partials that
// gsa_decode keeps in the caller's workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never uses the
// array's name as an address: its device address is looked up once per device
// and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)GSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call on that device, with it current); nullptr and the HIP error on failure.
void* scratch_address(int dev, hipError_t* err) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = p;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t gsa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

gsa_status gsa_decode_noalloc(const void* Q, const void* Kc, const void* Vc, const float* G, void* Y, int64_t B,
                              int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int mode, int dtype, int num_splits,
                              void* stream) {
  const char* fn = "gsa_decode_noalloc";
  if (!Q || !Kc || !Vc || !Y) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (gsa_status st = check_attn_shape(fn, B, L, Hq, Hkv, D, mode, G, 1)) return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (num_splits < 0) return fail(GSA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  if (!prod_le({B, L}, kIntMax)) return fail(GSA_ERR_UNSUPPORTED, "%s: B*L exceeds the supported range", fn);
  if (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(Y) || (G && !aligned16(G)))
    return fail(GSA_ERR_MISALIGNED, "%s: Q, Kc, Vc, G and Y must be 16-byte aligned", fn);
  int64_t ns = 0;
  if (dtype == GSA_BF16) {
    ns = gsa_decode_num_splits(B, L, Hq, Hkv, D, num_splits);
    const size_t need = gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits);
    if (need > kNoAllocScratchBytes)
      return fail(GSA_ERR_WORKSPACE,
                  "%s: these sizes need %zu bytes of split partials, more than the %zu-byte device scratch "
                  "(fewer splits or a smaller batch fit; gsa_decode takes a caller workspace of any size)",
                  fn, need, kNoAllocScratchBytes);
  }
  if (gsa_status st = check_device()) return st;
  if (dtype != GSA_BF16)  // float32 decode needs no scratch
    return hip_result(gsa::launch_attn_fwd(Q, Kc, Vc, G, Y, nullptr, (int)B, 1, (int)L, (int)Hq, (int)Hkv, (int)D,
                                           mode, false, (hipStream_t)stream),
                      fn);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(GSA_ERR_NO_DEVICE, "%s: hipGetDevice failed", fn);
  }
  hipError_t e = hipSuccess;
  void* ws = scratch_address(dev, &e);
  if (ws == nullptr) return fail(GSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
  return hip_result(gsa::launch_decode_bf16(Q, Kc, Vc, G, Y, ws, (int)B, (int)L, (int)Hq, (int)Hkv, (int)D, mode,
                                            (int)ns, (hipStream_t)stream),
                    fn);
}

}  // extern "C"

namespace {
// gsa_gated_decode's workspace: [decode partials | split-K gate parts | G],
// each 256-byte aligned (the gate parts only when gsa_gate_logits_ws takes its
// split-K path).
struct GatedDecodePlan {
  size_t dec_bytes = 0, gws_off = 0, gws_bytes = 0, g_off = 0, total = 0;
};
GatedDecodePlan gated_decode_plan(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t d_model,
                                  int mode, int dtype, int num_splits) {
  GatedDecodePlan p;
  if (dtype == GSA_BF16) p.dec_bytes = gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits);
  size_t off = (p.dec_bytes + 255) & ~(size_t)255;
  if (mode != GSA_GATE_NONE) {
    const int64_t N = mode == GSA_GATE_HEADWISE ? Hq : Hq * D;
    p.gws_off = off;
    p.gws_bytes = gsa_gate_logits_workspace_bytes(B, d_model, N, dtype);
    off += (p.gws_bytes + 255) & ~(size_t)255;
    p.g_off = off;
    off += (size_t)(B * N) * sizeof(float);
  }
  p.total = off;
  return p;
}
}  // namespace

extern "C" {

size_t gsa_gated_decode_workspace_bytes(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t d_model,
                                        int mode, int dtype, int num_splits) {
  if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || num_splits < 0) return 0;
  if (mode != GSA_GATE_NONE && mode != GSA_GATE_ELEMENTWISE && mode != GSA_GATE_HEADWISE) return 0;
  if (mode != GSA_GATE_NONE && (d_model <= 0 || d_model > kIntMax)) return 0;
  if (!prod_le({B, L}, kIntMax) || Hq > 4096 || D > 4096) return 0;
  if (mode != GSA_GATE_NONE && (!prod_le({B, Hq, D, 16}, kElemMax) || !prod_le({B, d_model}, kElemMax) ||
                                 !prod_le({d_model, Hq, D}, kElemMax)))
    return 0;
  return gated_decode_plan(B, L, Hq, Hkv, D, d_model, mode, dtype, num_splits).total;
}

gsa_status gsa_gated_decode(const void* X, const void* W, const void* Q, const void* Kc, const void* Vc, void* Y,
                            int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t d_model, int mode,
                            int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gsa_gated_decode";
  const bool gated = mode != GSA_GATE_NONE;
  if (!Q || !Kc || !Vc || !Y) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (gated != (X != nullptr) || gated != (W != nullptr))
    return fail(GSA_ERR_INVALID_ARG, "%s: X and W must be given exactly when a gate is", fn);
  // the shape rules of gsa_decode (checked with a stand-in gate pointer)
  if (gsa_status st = check_attn_shape(fn, B, L, Hq, Hkv, D, mode, gated ? (const float*)W : nullptr, 1)) return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (num_splits < 0) return fail(GSA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  if (!prod_le({B, L}, kIntMax)) return fail(GSA_ERR_UNSUPPORTED, "%s: B*L exceeds the supported range", fn);
  if (gated && (d_model <= 0 || d_model > kIntMax))
    return fail(GSA_ERR_INVALID_ARG, "%s: d_model=%lld must be positive", fn, (long long)d_model);
  if (gated && d_model % 8 != 0)
    return fail(GSA_ERR_UNSUPPORTED, "%s: d_model=%lld is not a multiple of 8", fn, (long long)d_model);
  if (gated && (!prod_le({B, Hq, D, 16}, kElemMax) || !prod_le({B, d_model}, kElemMax) ||
                !prod_le({d_model, Hq, D}, kElemMax)))
    return fail(GSA_ERR_UNSUPPORTED, "%s: sizes exceed the supported range", fn);
  if (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(Y) || (X && !aligned16(X)) ||
      (W && !aligned16(W)))
    return fail(GSA_ERR_MISALIGNED, "%s: X, W, Q, Kc, Vc and Y must be 16-byte aligned", fn);
  const GatedDecodePlan plan = gated_decode_plan(B, L, Hq, Hkv, D, d_model, mode, dtype, num_splits);
  if (plan.total > 0 && (workspace == nullptr || workspace_bytes < plan.total))
    return fail(GSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, plan.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (workspace && !aligned16(workspace)) return fail(GSA_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  char* ws = (char*)workspace;
  // bf16, elementwise, split-K gate: its partial logits go to the workspace and
  // the decode merge adds them and applies σ (one launch fewer than the part
  // sum kernel; the same operations in the same order)
  if (dtype == GSA_BF16 && mode == GSA_GATE_ELEMENTWISE && plan.gws_bytes > 0) {
    const int64_t N = Hq * D;
    const int64_t gs = gsa::gate_splitk_splits(B, d_model, N);
    float* gparts = (float*)(ws + plan.gws_off);
    hipError_t e = gsa::launch_gate_gemm_splitk_parts(X, W, gparts, B, d_model, N, (hipStream_t)stream);
    if (e != hipSuccess) return hip_result(e, fn);
    const int64_t ns = gsa_decode_num_splits(B, L, Hq, Hkv, D, num_splits);
    return hip_result(gsa::launch_decode_gateparts_bf16(Q, Kc, Vc, gparts, (int)gs, Y, ws, (int)B, (int)L, (int)Hq,
                                                        (int)Hkv, (int)D, (int)ns, (hipStream_t)stream),
                      fn);
  }
  // otherwise the gate into the workspace, then the decode
  float* G = gated ? (float*)(ws + plan.g_off) : nullptr;
  if (gated) {
    const int64_t N = mode == GSA_GATE_HEADWISE ? Hq : Hq * D;
    gsa_status s1 = gsa_gate_logits_ws(X, W, G, B, d_model, N, dtype, GSA_ACT_SIGMOID,
                                       plan.gws_bytes > 0 ? ws + plan.gws_off : nullptr, plan.gws_bytes, stream);
    if (s1 != GSA_OK) return s1;
  }
  return gsa_decode(Q, Kc, Vc, G, Y, B, L, Hq, Hkv, D, mode, dtype, num_splits, ws, plan.dec_bytes, stream);
}

gsa_status gsa_decode_variant(const void* Q, const void* Kc, const void* Vc, const float* G, void* Y, int64_t B,
                              int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int layout, int combine, int norm,
                              int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gsa_decode_variant";
  if (!Q || !Kc || !Vc || !Y) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (layout < GSA_GATE_NONE || layout > GSA_GATE_SHARED)
    return fail(GSA_ERR_INVALID_ARG, "%s: unknown gate layout %d", fn, layout);
  if (combine != GSA_COMBINE_MUL && combine != GSA_COMBINE_ADD)
    return fail(GSA_ERR_INVALID_ARG, "%s: unknown combine %d", fn, combine);
  if (norm != GSA_NORM_NONE && norm != GSA_NORM_RMS) return fail(GSA_ERR_INVALID_ARG, "%s: unknown norm %d", fn, norm);
  // the shape rules of gsa_decode, with the shared layout checked as a gate
  if (gsa_status st = check_attn_shape(fn, B, L, Hq, Hkv, D,
                                       layout == GSA_GATE_SHARED ? GSA_GATE_ELEMENTWISE : layout, G, 1))
    return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (num_splits < 0) return fail(GSA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  if (!prod_le({B, L}, kIntMax)) return fail(GSA_ERR_UNSUPPORTED, "%s: B*L exceeds the supported range", fn);
  if (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(Y) || (G && !aligned16(G)))
    return fail(GSA_ERR_MISALIGNED, "%s: Q, Kc, Vc, G and Y must be 16-byte aligned", fn);
  int64_t ns = 0;
  if (dtype == GSA_BF16) {
    ns = gsa_decode_num_splits(B, L, Hq, Hkv, D, num_splits);
    const size_t need = gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits);
    if (workspace_bytes < need || (need > 0 && workspace == nullptr))
      return fail(GSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
    if (workspace && !aligned16(workspace)) return fail(GSA_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
  }
  if (gsa_status st = check_device()) return st;
  const int add = combine == GSA_COMBINE_ADD, rms = norm == GSA_NORM_RMS;
  if (dtype == GSA_BF16)
    return hip_result(gsa::launch_decode_variant_bf16(Q, Kc, Vc, G, Y, workspace, (int)B, (int)L, (int)Hq,
                                                      (int)Hkv, (int)D, layout, add, rms, (int)ns,
                                                      (hipStream_t)stream),
                      fn);
  return hip_result(gsa::launch_attn_fwd_variant_f32_decode(Q, Kc, Vc, G, Y, (int)B, (int)L, (int)Hq, (int)Hkv,
                                                            (int)D, layout, add, rms, (hipStream_t)stream),
                    fn);
}

}  // extern "C"

namespace {
// gsa_backward's side stream: when the key/value grid is not cut into GQA
// slices, dQ and then dX run on it beside dK/dV and dW, which stay on the
// caller's stream.  One per device, created on the device's first backward
// call with default priority, with the fork and join events; the mutex keeps
// each call's record/wait pairs together when several host threads use one
// device.  A stream being captured into a graph gets the sequential order
// instead (no side stream is created or joined while capturing).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipError_t err = hipSuccess;
  std::mutex mu;
};
std::once_flag g_side_once[kMaxDevices];
SideStream g_side[kMaxDevices];

SideStream* side_stream(int dev) {
  std::call_once(g_side_once[dev], [dev] {
    SideStream& ss = g_side[dev];
    hipError_t e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) (void)hipGetLastError();
    ss.err = e;
  });
  return g_side[dev].err == hipSuccess ? &g_side[dev] : nullptr;
}

// Workspace of gsa_backward, each region 256-byte aligned:
//   dY  = dY' ⊙ g                 bf16 [B, S, Hq, D]          (gated modes)
//   per-row statistics            fp32 2 x [B*Hq, Sp]          (base-2 LSE, then D; Sp = S rounded up to 64)
//   dZ                            bf16 [B*S, N]                (gated modes)
//   partial sums                  fp32, the larger of
//       dK, dV slices             2 x [slices, B, S, Hkv, D]   (when a GQA group is split)
//       dW_θ token chunks         [splits, d_model, N]         (gated modes, splits > 1)
//   (both partial sets are consumed before the next kernel on the stream starts,
//   so they share one region)
struct BwdLayout {
  size_t dy = 0, stat = 0, dz = 0, part = 0, total = 0;
  int64_t splits = 1;
};
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
BwdLayout bwd_layout(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t d_model, int mode) {
  BwdLayout l;
  const bool gated = mode != GSA_GATE_NONE;
  const int64_t M = B * S, N = mode == GSA_GATE_HEADWISE ? Hq : Hq * D;
  size_t off = 0;
  l.dy = off;
  if (gated) off += align256((size_t)(M * Hq * D) * 2);
  l.stat = off;
  off += align256((size_t)(2 * B * Hq * gsa::bwd_stat_rows((int)S)) * 4);
  l.dz = off;
  if (gated) off += align256((size_t)(M * N) * 2);
  l.part = off;
  size_t part = 0;
  const int64_t ns = gsa::bwd_kv_slices((int)B, (int)S, (int)Hq, (int)Hkv, (int)D);
  if (ns > 1) part = (size_t)(2 * ns * M * Hkv * D) * 4;
  if (gated) {
    l.splits = gsa::bwd_dw_splits(M, d_model, N);
    if (l.splits > 1) part = std::max(part, (size_t)(l.splits * d_model * N) * 4);
  }
  off += align256(part);
  l.total = off;
  return l;
}
constexpr int64_t kU32Bytes = 0xfffffff0LL;   // operands addressed with 32-bit byte offsets
}  // namespace

extern "C" {

size_t gsa_backward_workspace_bytes(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                    int64_t d_model, int mode) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return 0;
  if (mode != GSA_GATE_NONE && mode != GSA_GATE_ELEMENTWISE && mode != GSA_GATE_HEADWISE) return 0;
  if (mode != GSA_GATE_NONE && d_model <= 0) return 0;
  if (!prod_le({B, S}, kIntMax) || Hq > 4096 || D > 128 || d_model > kIntMax) return 0;
  return bwd_layout(B, S, Hq, Hkv, D, d_model, mode).total;
}

gsa_status gsa_backward(const void* X, const void* W, const float* G, const void* Q, const void* K,
                        const void* V, const void* Y, const float* LSE, const void* dY, void* dX,
                        float* dW, void* dQ, void* dK, void* dV, int64_t B, int64_t S, int64_t Hq,
                        int64_t Hkv, int64_t D, int64_t d_model, int mode, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const char* fn = "gsa_backward";
  if (!Q || !K || !V || !Y || !LSE || !dY || !dQ || !dK || !dV)
    return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (gsa_status st = check_attn_shape(fn, B, S, Hq, Hkv, D, mode, G)) return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (dtype != GSA_BF16) return fail(GSA_ERR_UNSUPPORTED, "%s: only GSA_BF16 is supported", fn);
  const bool gated = mode != GSA_GATE_NONE;
  if (gated != (X != nullptr) || gated != (W != nullptr) || gated != (dX != nullptr) || gated != (dW != nullptr))
    return fail(GSA_ERR_INVALID_ARG, "%s: X, W, dX and dW must be given exactly when a gate is", fn);
  const int64_t M = B * S, N = mode == GSA_GATE_HEADWISE ? Hq : Hq * D;
  if (gated) {
    if (d_model <= 0 || d_model > kIntMax)
      return fail(GSA_ERR_INVALID_ARG, "%s: d_model=%lld must be positive", fn, (long long)d_model);
    if (d_model % 8 != 0 || N % 8 != 0)
      return fail(GSA_ERR_UNSUPPORTED, "%s: d_model=%lld and the gate width %lld must be multiples of 8", fn,
                  (long long)d_model, (long long)N);
    if (!prod_le({M, d_model, 2}, kU32Bytes) || !prod_le({M, N, 2}, kU32Bytes) || !prod_le({d_model, N, 4}, kU32Bytes))
      return fail(GSA_ERR_UNSUPPORTED, "%s: X, dZ or W_theta exceeds 4 GiB", fn);
  }
  const void* ptrs[] = {X, W, G, Q, K, V, Y, dY, dX, dW, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p))
      return fail(GSA_ERR_MISALIGNED, "%s: every tensor and the workspace must be 16-byte aligned", fn);
  if (((uintptr_t)LSE % 4) != 0) return fail(GSA_ERR_MISALIGNED, "%s: LSE must be 4-byte aligned", fn);
  const BwdLayout lay = bwd_layout(B, S, Hq, Hkv, D, d_model, mode);
  if (workspace == nullptr || workspace_bytes < lay.total)
    return fail(GSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, lay.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (gsa_status st = check_device()) return st;
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  void* dz = gated ? ws + lay.dz : nullptr;
  // dQ (then dX) on the side stream beside dK/dV (then dW) when the key/value
  // grid is not sliced: the sliced grid and the dW token chunks share the
  // partial-sum region, and the sliced (GQA) shapes ran slower that way
  SideStream* side = nullptr;
  if (gsa::bwd_kv_slices((int)B, (int)S, (int)Hq, (int)Hkv, (int)D) == 1) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess) {
      (void)hipGetLastError();
      cap = hipStreamCaptureStatusActive;   // unknown: stay on one stream
    }
    int dev = -1;
    if (cap == hipStreamCaptureStatusNone && hipGetDevice(&dev) == hipSuccess) side = side_stream(dev);
  }
  std::unique_lock<std::mutex> lock;
  if (side) lock = std::unique_lock<std::mutex>(side->mu);
  hipStream_t st2 = side ? side->s : st;
  const char* what = "gsa_backward attention launch";
  hipError_t e = gsa::launch_attn_bwd(Q, K, V, dY, Y, G, LSE, dQ, dK, dV, gated ? ws + lay.dy : nullptr,
                                      (float*)(ws + lay.stat), dz, (float*)(ws + lay.part), (int)B, (int)S,
                                      (int)Hq, (int)Hkv, (int)D, mode, st, st2, side ? side->fork : nullptr);
  if (e == hipSuccess && gated) {
    what = "gsa_backward dX launch";
    e = gsa::launch_bwd_gemm_dx(dz, W, dX, M, d_model, N, st2);
    if (e == hipSuccess) {
      what = "gsa_backward dW launch";
      e = gsa::launch_bwd_gemm_dw(X, dz, dW, (float*)(ws + lay.part), M, d_model, N, lay.splits, st);
    }
  }
  if (side) {   // the caller's stream waits for whatever the side stream got (also after an error)
    hipError_t ej = hipEventRecord(side->join, st2);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(st, side->join, 0);
    if (e == hipSuccess && ej != hipSuccess) {
      e = ej;
      what = "gsa_backward join";
    }
  }
  if (e != hipSuccess) return hip_result(e, what);
  return ok();
}

gsa_status gsa_project_qkvg(const void* X, const void* W, void* Q, void* K, void* V, float* G, int64_t M,
                            int64_t d_model, int64_t Hq, int64_t Hkv, int64_t D, int64_t n_gate, int dtype,
                            void* stream) {
  const char* fn = "gsa_project_qkvg";
  if (!X || !W || !Q || !K || !V) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (M <= 0 || d_model <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || n_gate < 0)
    return fail(GSA_ERR_INVALID_ARG, "%s: sizes must be positive (n_gate >= 0)", fn);
  if (Hq % Hkv != 0)
    return fail(GSA_ERR_INVALID_ARG, "%s: Hq=%lld is not a multiple of Hkv=%lld", fn, (long long)Hq,
                (long long)Hkv);
  if ((n_gate == 0) != (G == nullptr))
    return fail(GSA_ERR_INVALID_ARG, "%s: G must be NULL exactly when n_gate is 0", fn);
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (dtype != GSA_BF16) return fail(GSA_ERR_UNSUPPORTED, "%s: only GSA_BF16 is supported", fn);
  if (Hq > 4096 || D > 4096 || n_gate > kIntMax)
    return fail(GSA_ERR_UNSUPPORTED, "%s: sizes exceed the supported range", fn);
  const int64_t nq = Hq * D, nkv = Hkv * D, N = nq + 2 * nkv + n_gate;
  if (d_model % 8 != 0 || nq % 8 != 0 || nkv % 8 != 0 || n_gate % 8 != 0)
    return fail(GSA_ERR_UNSUPPORTED, "%s: d_model and every output width must be multiples of 8", fn);
  if (!prod_le({M, d_model, 2}, kIntMax - 1) || !prod_le({d_model, N, 2}, kIntMax - 1))
    return fail(GSA_ERR_UNSUPPORTED, "%s: X or W exceeds 2 GiB", fn);
  if (!aligned16(X) || !aligned16(W) || !aligned16(Q) || !aligned16(K) || !aligned16(V) || (G && !aligned16(G)))
    return fail(GSA_ERR_MISALIGNED, "%s: X, W, Q, K, V and G must be 16-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_project_qkvg(X, W, Q, K, V, G, M, d_model, nq, nkv, n_gate, (hipStream_t)stream),
                    fn);
}

gsa_status gsa_forward_variant(const void* Q, const void* K, const void* V, const float* G, void* Y,
                               float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                               int layout, int combine, int norm, int dtype, void* stream) {
  const char* fn = "gsa_forward_variant";
  if (!Q || !K || !V || !Y) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (layout < GSA_GATE_NONE || layout > GSA_GATE_SHARED)
    return fail(GSA_ERR_INVALID_ARG, "%s: unknown gate layout %d", fn, layout);
  if (combine != GSA_COMBINE_MUL && combine != GSA_COMBINE_ADD)
    return fail(GSA_ERR_INVALID_ARG, "%s: unknown combine %d", fn, combine);
  if (norm != GSA_NORM_NONE && norm != GSA_NORM_RMS)
    return fail(GSA_ERR_INVALID_ARG, "%s: unknown norm %d", fn, norm);
  // the shape rules of gsa_forward, with the shared layout checked as a gate
  if (gsa_status st = check_attn_shape(fn, B, S, Hq, Hkv, D, layout == GSA_GATE_SHARED ? GSA_GATE_ELEMENTWISE
                                                                                        : layout, G))
    return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Y) || (G && !aligned16(G)))
    return fail(GSA_ERR_MISALIGNED, "%s: Q, K, V, G and Y must be 16-byte aligned", fn);
  if (LSE && ((uintptr_t)LSE % 4) != 0) return fail(GSA_ERR_MISALIGNED, "%s: LSE must be 4-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_attn_fwd_variant(Q, K, V, G, Y, LSE, (int)B, (int)S, (int)Hq, (int)Hkv, (int)D,
                                                 layout, combine == GSA_COMBINE_ADD, norm == GSA_NORM_RMS,
                                                 dtype == GSA_BF16, (hipStream_t)stream),
                    fn);
}

gsa_status gsa_forward_value_gated(const void* Q, const void* K, const void* V, const float* Gv, void* Y,
                                   float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                   int layout, int dtype, void* stream) {
  const char* fn = "gsa_forward_value_gated";
  if (!Q || !K || !V || !Gv || !Y) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (layout != GSA_GATE_ELEMENTWISE && layout != GSA_GATE_HEADWISE)
    return fail(GSA_ERR_INVALID_ARG, "%s: layout must be GSA_GATE_ELEMENTWISE or GSA_GATE_HEADWISE", fn);
  // the shape rules of gsa_forward (the value gate is checked like an output gate)
  if (gsa_status st = check_attn_shape(fn, B, S, Hq, Hkv, D, layout, Gv)) return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Y) || !aligned16(Gv))
    return fail(GSA_ERR_MISALIGNED, "%s: Q, K, V, Gv and Y must be 16-byte aligned", fn);
  if (LSE && ((uintptr_t)LSE % 4) != 0) return fail(GSA_ERR_MISALIGNED, "%s: LSE must be 4-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_attn_fwd_value_gated(Q, K, V, Gv, Y, LSE, (int)B, (int)S, (int)Hq, (int)Hkv, (int)D,
                                                     layout == GSA_GATE_HEADWISE, dtype == GSA_BF16,
                                                     (hipStream_t)stream),
                    fn);
}

gsa_status gsa_value_gate(const void* V, const float* G, void* Vout, int64_t B, int64_t S, int64_t Hkv,
                          int64_t D, int layout, int dtype, void* stream) {
  const char* fn = "gsa_value_gate";
  if (!V || !G || !Vout) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B <= 0 || S <= 0 || Hkv <= 0 || D <= 0) return fail(GSA_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
  if (layout != GSA_GATE_ELEMENTWISE && layout != GSA_GATE_HEADWISE)
    return fail(GSA_ERR_INVALID_ARG, "%s: layout must be GSA_GATE_ELEMENTWISE or GSA_GATE_HEADWISE", fn);
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (D != 64 && D != 128) return fail(GSA_ERR_UNSUPPORTED, "%s: head dim %lld is not 64 or 128", fn, (long long)D);
  if (!prod_le({B, S}, kIntMax) || !prod_le({B, S, Hkv, D}, kElemMax))
    return fail(GSA_ERR_UNSUPPORTED, "%s: sizes exceed the supported range", fn);
  if (!aligned16(V) || !aligned16(G) || !aligned16(Vout))
    return fail(GSA_ERR_MISALIGNED, "%s: V, G and Vout must be 16-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_value_gate(V, G, Vout, B * S, (int)Hkv, (int)D, layout == GSA_GATE_HEADWISE,
                                           dtype == GSA_BF16, (hipStream_t)stream),
                    fn);
}

gsa_status gsa_gate_head_mean(const float* G, float* Gs, int64_t M, int64_t Hq, int64_t D, void* stream) {
  const char* fn = "gsa_gate_head_mean";
  if (!G || !Gs) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (M <= 0 || Hq <= 0 || D <= 0)
    return fail(GSA_ERR_INVALID_ARG, "%s: sizes must be positive (M=%lld Hq=%lld D=%lld)", fn, (long long)M,
                (long long)Hq, (long long)D);
  if (D % 4 != 0) return fail(GSA_ERR_UNSUPPORTED, "%s: D=%lld is not a multiple of 4", fn, (long long)D);
  if (Hq > 4096 || D > 4096 || M > kIntMax || !prod_le({M, Hq, D}, kElemMax))
    return fail(GSA_ERR_UNSUPPORTED, "%s: sizes exceed the supported range", fn);
  if (!aligned16(G) || !aligned16(Gs)) return fail(GSA_ERR_MISALIGNED, "%s: G and Gs must be 16-byte aligned", fn);
  const uintptr_t g0 = (uintptr_t)G, g1 = g0 + (uintptr_t)(M * Hq * D) * 4;
  const uintptr_t s0 = (uintptr_t)Gs, s1 = s0 + (uintptr_t)(M * D) * 4;
  if (s0 < g1 && g0 < s1) return fail(GSA_ERR_INVALID_ARG, "%s: G and Gs may not overlap", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_gate_head_mean(G, Gs, M, (int)Hq, (int)D, (hipStream_t)stream), fn);
}

gsa_status gsa_first_token_attention(const void* Q, const void* K, const float* LSE, float* F,
                                     float* head_mean, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                     int64_t D, int dtype, void* stream) {
  const char* fn = "gsa_first_token_attention";
  if (!Q || !K || !LSE || !F) return fail(GSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (gsa_status st = check_attn_shape(fn, B, S, Hq, Hkv, D, GSA_GATE_NONE, nullptr)) return st;
  if (gsa_status st = check_dtype(fn, dtype)) return st;
  if (!aligned16(Q) || !aligned16(K)) return fail(GSA_ERR_MISALIGNED, "%s: Q and K must be 16-byte aligned", fn);
  if (((uintptr_t)LSE | (uintptr_t)F | (uintptr_t)head_mean) % 4 != 0)
    return fail(GSA_ERR_MISALIGNED, "%s: LSE, F and head_mean must be 4-byte aligned", fn);
  if (gsa_status st = check_device()) return st;
  return hip_result(gsa::launch_first_token_share(Q, K, LSE, F, head_mean, (int)B, (int)S, (int)Hq, (int)Hkv,
                                                  (int)D, dtype == GSA_BF16, (hipStream_t)stream),
                    fn);
}

}  // extern "C"
