// C ABI of libsparge.so (declared in include/sparge.h): argument checks on
// the host, sizes, and dispatch to the kernels on the caller's stream.
#include <math.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/sparge.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s", where, hipGetErrorString(e));
  g_last_error = buf;
  return SPARGE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Shape checks common to every entry point. Returns SPARGE_OK or an error.
int check_shape(int B, int H, int N, int d, int block_q, int block_k) {
  if (B < 1 || H < 1 || N < 1) return fail(SPARGE_ERR_INVALID_ARG, "B, H and N must be >= 1");
  // block counts are formed as (N + size - 1) / size in 32-bit arithmetic
  if (N > 0x7FFFFFFF - 1024) return fail(SPARGE_ERR_INVALID_ARG, "N too large");
  if (d != 64 && d != 128) return fail(SPARGE_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (block_q != 64 && block_q != 128)
    return fail(SPARGE_ERR_UNSUPPORTED, "block_q must be 64 or 128");
  if (block_k != 64) return fail(SPARGE_ERR_UNSUPPORTED, "block_k must be 64");
  // every element offset must fit comfortably in 64-bit arithmetic and
  // every workgroup count in a 32-bit grid dimension
  const double elems = (double)B * H * (double)N * d;
  if (elems > 9.0e15) return fail(SPARGE_ERR_INVALID_ARG, "tensor too large");
  const double tiles = (double)B * H * ceil_div(N, block_q);
  if (tiles > 2.0e9) return fail(SPARGE_ERR_INVALID_ARG, "too many query blocks");
  return SPARGE_OK;
}

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

constexpr int kMaxKeyBlocks = 4096;  // sort capacity of the selection kernel

size_t mask_ws(int B, int H, int N, int d, int block_q, int block_k) {
  const size_t BH = (size_t)B * H;
  const size_t n_q = ceil_div(N, block_q), n_k = ceil_div(N, block_k);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up(BH * n_q * d * sizeof(double)) + up(BH * n_k * d * sizeof(double)) +
         up(BH * n_q * n_k * sizeof(double));
}

// the routed mask adds the transposed float64 weights and the projected means
size_t routed_mask_ws(int B, int H, int N, int d, int block_q, int block_k) {
  const size_t BH = (size_t)B * H;
  const size_t n_q = ceil_div(N, block_q), n_k = ceil_div(N, block_k);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return mask_ws(B, H, N, d, block_q, block_k) + 2 * up(BH * d * d * sizeof(double)) +
         up(BH * n_q * d * sizeof(double)) + up(BH * n_k * d * sizeof(double));
}

int check_attn_args(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                    const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                    int block_k, float scale, const void* o) {
  int rc = check_shape(B, H, N, d, block_q, block_k);
  if (rc != SPARGE_OK) return rc;
  if (!q || !k || !v || !o || !kv_idx || !kv_cnt)
    return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SPARGE_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (!aligned(kv_idx, 4) || !aligned(kv_cnt, 4))
    return fail(SPARGE_ERR_INVALID_ARG, "kv_idx and kv_cnt must be 4-byte aligned");
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(SPARGE_ERR_INVALID_ARG, "scale must be finite and > 0");
  return SPARGE_OK;
}

}  // namespace

extern "C" {

const char* sparge_last_error(void) { return g_last_error.c_str(); }

size_t sparge_mask_workspace_bytes(int B, int H, int N, int d, int block_q, int block_k) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, block_q, block_k);
  g_last_error = saved;
  if (rc != SPARGE_OK || ceil_div(N, block_k) > kMaxKeyBlocks) return 0;
  return mask_ws(B, H, N, d, block_q, block_k);
}

}  // extern "C"

namespace {
// the mask, optionally with the router's projections (wq, wk both set);
// phase 1 pools only (q, k, workspace), phase 2 does the rest (workspace and
// outputs), phase 0 both
int mask_impl(const void* q, const void* k, const float* wq, const float* wk, int B, int H,
              int N, int d, int block_q, int block_k, float k_frac, float p_mass, float scale,
              uint32_t* mask_bits, int32_t* kv_idx, int32_t* kv_cnt, double* block_logits,
              void* workspace, size_t workspace_bytes, void* stream, int phase = 0,
              bool launch = true, void* lowbit_ws = nullptr, size_t lowbit_ws_bytes = 0) {
  int rc = check_shape(B, H, N, d, block_q, block_k);
  if (rc != SPARGE_OK) return rc;
  const int n_q = ceil_div(N, block_q), n_k = ceil_div(N, block_k);
  if (n_k > kMaxKeyBlocks)
    return fail(SPARGE_ERR_UNSUPPORTED, "more than 4096 key blocks (N > 262144)");
  const bool pools = phase != 2, selects = phase != 1;
  if (selects) {
    if (!(k_frac > 0.0f) || !(k_frac <= 1.0f))
      return fail(SPARGE_ERR_INVALID_ARG, "k_frac must satisfy 0 < k_frac <= 1");
    if (!(p_mass >= 0.0f) || !isfinite(p_mass))
      return fail(SPARGE_ERR_INVALID_ARG, "p_mass must be finite and >= 0");
    if (!(scale > 0.0f) || !isfinite(scale))
      return fail(SPARGE_ERR_INVALID_ARG, "scale must be finite and > 0");
  }
  if ((pools && (!q || !k)) || (selects && (!mask_bits || !kv_idx || !kv_cnt)) || !workspace)
    return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if ((pools && (!aligned(q, 16) || !aligned(k, 16))) || !aligned(workspace, 16))
    return fail(SPARGE_ERR_INVALID_ARG, "q, k and workspace must be 16-byte aligned");
  if (selects && (!aligned(mask_bits, 4) || !aligned(kv_idx, 4) || !aligned(kv_cnt, 4)))
    return fail(SPARGE_ERR_INVALID_ARG, "mask_bits, kv_idx, kv_cnt must be 4-byte aligned");
  if (selects && block_logits && !aligned(block_logits, 8))
    return fail(SPARGE_ERR_INVALID_ARG, "block_logits must be 8-byte aligned");
  const bool routed = wq != nullptr;
  if (routed && (!aligned(wq, 4) || !aligned(wk, 4)))
    return fail(SPARGE_ERR_INVALID_ARG, "w_q and w_k must be 4-byte aligned");
  // scores written to the caller's block_logits need no room in the workspace
  const size_t BH_ = (size_t)B * H;
  const size_t score_bytes = (BH_ * n_q * n_k * sizeof(double) + 255) & ~(size_t)255;
  const size_t need = routed ? routed_mask_ws(B, H, N, d, block_q, block_k)
                      : (block_logits && selects) ? mask_ws(B, H, N, d, block_q, block_k) - score_bytes
                                                  : mask_ws(B, H, N, d, block_q, block_k);
  if (workspace_bytes < need) return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  if (lowbit_ws) {  // the pooling pass also writes the low-bit codes of Q and K
    if (!aligned(lowbit_ws, 256))
      return fail(SPARGE_ERR_INVALID_ARG, "lowbit_workspace must be 256-byte aligned");
    if (lowbit_ws_bytes < sparge::lowbit_workspace_bytes(B, H, N, d, block_q))
      return fail(SPARGE_ERR_INVALID_ARG, "lowbit_workspace too small");
  }
  if (!launch) return SPARGE_OK;  // arguments checked only

  sparge::MaskLaunch a{};
  a.phase = phase;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q; a.block_k = block_k;
  a.n_q = n_q; a.n_k = n_k;
  a.npad = next_pow2(n_k < 64 ? 64 : n_k);
  a.words = ceil_div(n_k, 32);
  // Top-k size from the float32 fraction, evaluated in double
  const double kk = ceil((double)k_frac * n_k - 1e-6);
  a.K_k = (int)fmin((double)n_k, fmax(1.0, kk));
  a.keep_all = p_mass >= 1.0f;
  a.p = (double)p_mass;
  a.scale = (double)scale;
  const size_t BH = (size_t)B * H;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.qbar = reinterpret_cast<double*>(ws);
  a.kbar = reinterpret_cast<double*>(ws + up(BH * n_q * d * sizeof(double)));
  a.logits = block_logits
                 ? block_logits
                 : reinterpret_cast<double*>(ws + up(BH * n_q * d * sizeof(double)) +
                                             up(BH * n_k * d * sizeof(double)));
  if (routed) {  // after the plain layout: W_q^T, W_k^T, projected Qbar, Kbar
    unsigned char* r = ws + mask_ws(B, H, N, d, block_q, block_k);
    a.wq = wq;
    a.wk = wk;
    a.wqT = reinterpret_cast<double*>(r);
    a.wkT = reinterpret_cast<double*>(r + up(BH * d * d * sizeof(double)));
    a.qbar_p = reinterpret_cast<double*>(r + 2 * up(BH * d * d * sizeof(double)));
    a.kbar_p = reinterpret_cast<double*>(r + 2 * up(BH * d * d * sizeof(double)) +
                                         up(BH * n_q * d * sizeof(double)));
  }
  a.bits = mask_bits;
  a.idx = kv_idx;
  a.cnt = kv_cnt;
  if (lowbit_ws) {
    sparge::LowbitLaunch l{};
    l.B = B; l.H = H; l.N = N; l.d = d; l.block_q = block_q; l.n_q = n_q; l.n_k = n_k;
    sparge::lowbit_layout(l, static_cast<unsigned char*>(lowbit_ws));
    a.qc = l.qc; a.kc = l.kc; a.qsc = l.qs; a.ksc = l.ks;
  }
  const hipError_t e = sparge::launch_mask(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask prediction launch");
  return SPARGE_OK;
}
}  // namespace

extern "C" {

int sparge_mask_predict(const void* q, const void* k, int B, int H, int N, int d, int block_q,
                        int block_k, float k_frac, float p_mass, float scale,
                        uint32_t* mask_bits, int32_t* kv_idx, int32_t* kv_cnt,
                        double* block_logits, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_last_error.clear();
  return mask_impl(q, k, nullptr, nullptr, B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
                   mask_bits, kv_idx, kv_cnt, block_logits, workspace, workspace_bytes, stream);
}

int sparge_mask_pool(const void* q, const void* k, int B, int H, int N, int d, int block_q,
                     int block_k, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return mask_impl(q, k, nullptr, nullptr, B, H, N, d, block_q, block_k, 1.0f, 0.0f, 1.0f,
                   nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, 1);
}

int sparge_mask_pool_lowbit(const void* q, const void* k, int B, int H, int N, int d,
                            int block_q, int block_k, void* workspace, size_t workspace_bytes,
                            void* lowbit_workspace, size_t lowbit_workspace_bytes,
                            void* stream) {
  g_last_error.clear();
  if (!lowbit_workspace) return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  return mask_impl(q, k, nullptr, nullptr, B, H, N, d, block_q, block_k, 1.0f, 0.0f, 1.0f,
                   nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, 1,
                   true, lowbit_workspace, lowbit_workspace_bytes);
}

int sparge_mask_select(int B, int H, int N, int d, int block_q, int block_k, float k_frac,
                       float p_mass, float scale, uint32_t* mask_bits, int32_t* kv_idx,
                       int32_t* kv_cnt, double* block_logits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return mask_impl(nullptr, nullptr, nullptr, nullptr, B, H, N, d, block_q, block_k, k_frac,
                   p_mass, scale, mask_bits, kv_idx, kv_cnt, block_logits, workspace,
                   workspace_bytes, stream, 2);
}

size_t sparge_mask_routed_workspace_bytes(int B, int H, int N, int d, int block_q, int block_k) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, block_q, block_k);
  g_last_error = saved;
  if (rc != SPARGE_OK || ceil_div(N, block_k) > kMaxKeyBlocks) return 0;
  return routed_mask_ws(B, H, N, d, block_q, block_k);
}

int sparge_mask_predict_routed(const void* q, const void* k, const float* w_q, const float* w_k,
                               int B, int H, int N, int d, int block_q, int block_k,
                               float k_frac, float p_mass, float scale, uint32_t* mask_bits,
                               int32_t* kv_idx, int32_t* kv_cnt, double* block_logits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!w_q || !w_k) return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  return mask_impl(q, k, w_q, w_k, B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
                   mask_bits, kv_idx, kv_cnt, block_logits, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Mask prediction without a caller workspace. Its scratch (the pooled means
// and, unless the caller takes them, the block scores) lives in one
// file-scope device array per GPU, held from the library's first use on that
// GPU until the process ends. In host code `scratch` is only a stand-in for
// the symbol: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to the kernels.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;

std::once_flag g_scratch_once[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];

// this device's address of `scratch` (nullptr and a message on failure)
void* scratch_on_current_device(int* rc) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    *rc = fail(SPARGE_ERR_UNSUPPORTED, "device index above 63");
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
    *rc = hip_fail(g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev] : hipErrorUnknown,
                   "hipGetSymbolAddress(scratch)");
    return nullptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t sparge_mask_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int sparge_mask_predict_noalloc(const void* q, const void* k, int B, int H, int N, int d,
                                int block_q, int block_k, float k_frac, float p_mass,
                                float scale, uint32_t* mask_bits, int32_t* kv_idx,
                                int32_t* kv_cnt, double* block_logits, void* stream) {
  g_last_error.clear();
  int rc = check_shape(B, H, N, d, block_q, block_k);
  if (rc != SPARGE_OK) return rc;
  if (ceil_div(N, block_k) > kMaxKeyBlocks)
    return fail(SPARGE_ERR_UNSUPPORTED, "more than 4096 key blocks (N > 262144)");
  // the means always, the scores only when the caller does not take them
  const size_t BH = (size_t)B * H;
  const size_t n_q = ceil_div(N, block_q), n_k = ceil_div(N, block_k);
  const size_t need = block_logits ? mask_ws(B, H, N, d, block_q, block_k) -
                                         ((BH * n_q * n_k * sizeof(double) + 255) & ~(size_t)255)
                                   : mask_ws(B, H, N, d, block_q, block_k);
  if (need > kNoAllocScratchBytes) {
    char buf[200];
    snprintf(buf, sizeof buf,
             "this shape needs %zu bytes of scratch, more than the %zu bytes the "
             "no-allocation mask call holds (pass block_logits, or use "
             "sparge_mask_predict with a workspace)",
             need, kNoAllocScratchBytes);
    return fail(SPARGE_ERR_UNSUPPORTED, buf);
  }
  // every other argument is checked before any HIP call: a dry run against an
  // aligned stand-in for the scratch address
  rc = mask_impl(q, k, nullptr, nullptr, B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
                 mask_bits, kv_idx, kv_cnt, block_logits, reinterpret_cast<void*>(256),
                 kNoAllocScratchBytes, stream, 0, false);
  if (rc != SPARGE_OK) return rc;
  void* ws = scratch_on_current_device(&rc);
  if (!ws) return rc;
  return mask_impl(q, k, nullptr, nullptr, B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
                   mask_bits, kv_idx, kv_cnt, block_logits, ws, kNoAllocScratchBytes, stream);
}

size_t sparge_attn_workspace_bytes(int B, int H, int N, int d) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, 128, 64);
  g_last_error = saved;
  if (rc != SPARGE_OK) return 0;
  return sparge::attn_workspace_bytes(B, H, N, d);
}

namespace {
sparge::AttnLaunch attn_args(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                             const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                             int block_k, float scale, void* o, void* workspace) {
  sparge::AttnLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = kv_idx;
  a.cnt = kv_cnt;
  a.o = static_cast<uint16_t*>(o);
  a.vt = static_cast<uint16_t*>(workspace);
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q;
  a.n_q = ceil_div(N, block_q);
  a.n_k = ceil_div(N, block_k);
  a.scale = scale;
  return a;
}

int check_attn_workspace(const void* workspace, size_t workspace_bytes, int B, int H, int N,
                         int d) {
  if (!workspace) return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(workspace, 16))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < sparge::attn_workspace_bytes(B, H, N, d))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  return SPARGE_OK;
}
}  // namespace

int sparge_attn_fwd(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                    const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                    int block_k, float scale, void* o, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_last_error.clear();
  int rc = check_attn_args(q, k, v, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o);
  if (rc == SPARGE_OK) rc = check_attn_workspace(workspace, workspace_bytes, B, H, N, d);
  if (rc != SPARGE_OK) return rc;
  const sparge::AttnLaunch a =
      attn_args(q, k, v, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o, workspace);
  const hipError_t e = sparge::launch_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparge_attn_fwd launch");
  return SPARGE_OK;
}

int sparge_attn_fwd_lse(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                        const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                        int block_k, float scale, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_attn_args(q, k, v, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o);
  if (rc == SPARGE_OK) rc = check_attn_workspace(workspace, workspace_bytes, B, H, N, d);
  if (rc != SPARGE_OK) return rc;
  if (!lse || !aligned(lse, 4)) return fail(SPARGE_ERR_INVALID_ARG, "lse null or misaligned");
  sparge::AttnLaunch a =
      attn_args(q, k, v, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o, workspace);
  a.lse = lse;
  const hipError_t e = sparge::launch_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparge_attn_fwd_lse launch");
  return SPARGE_OK;
}

size_t sparge_attn_bwd_workspace_bytes(int B, int H, int N, int d, int block_q, int block_k) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, block_q, block_k);
  g_last_error = saved;
  if (rc != SPARGE_OK) return 0;
  return sparge::bwd_workspace_bytes(B, H, N, d, block_q);
}

}  // extern "C"

namespace {
// the backward, plain (alpha == nullptr) or with the linear branch
int bwd_impl(const char* name, int mode, const void* q, const void* k, const void* v,
             const void* o, const void* d_o, const float* lse, const int32_t* kv_idx,
             const int32_t* kv_cnt, const float* alpha, int B, int H, int N, int d, int block_q,
             int block_k, float scale, float drop_below, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_attn_args(q, k, v, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o);
  if (rc != SPARGE_OK) return rc;
  const bool linear = mode >= 0;
  if (!d_o || !lse || !dq || !dk || !dv || !workspace || (linear && !alpha))
    return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(d_o, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16) ||
      (linear && !aligned(alpha, mode == sparge::kLinMix ? 16 : 4)))
    return fail(SPARGE_ERR_INVALID_ARG, "d_o, dq, dk, dv, lse, alpha or workspace misaligned");
  if (workspace_bytes < sparge::bwd_workspace_bytes(B, H, N, d, block_q, linear))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  if (linear && block_q != d)
    return fail(SPARGE_ERR_UNSUPPORTED, "the linear branch is built for block_q == d (64 or 128)");
  if (linear && ceil_div(N, block_k) > kMaxKeyBlocks)
    return fail(SPARGE_ERR_UNSUPPORTED, "the linear backward supports at most 4096 key blocks");
  sparge::BwdLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dO = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.idx = kv_idx;
  a.cnt = kv_cnt;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q;
  a.n_q = ceil_div(N, block_q);
  a.n_k = ceil_div(N, block_k);
  a.scale = scale;
  a.workspace = static_cast<unsigned char*>(workspace);
  a.alpha = linear ? alpha : nullptr;
  a.lin_mode = linear ? mode : 0;
  a.drop_below = drop_below;
  const hipError_t e = sparge::launch_bwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, name);
  return SPARGE_OK;
}
}  // namespace

extern "C" {

int sparge_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                    const float* lse, const int32_t* kv_idx, const int32_t* kv_cnt, int B,
                    int H, int N, int d, int block_q, int block_k, float scale, void* dq,
                    void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl("sparge_attn_bwd launch", -1, q, k, v, o, d_o, lse, kv_idx, kv_cnt, nullptr, B,
                  H, N, d, block_q, block_k, scale, 0.0f, dq, dk, dv, workspace,
                  workspace_bytes, stream);
}

size_t sparge_attn_lowbit_workspace_bytes(int B, int H, int N, int d, int block_q, int block_k) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, block_q, block_k);
  g_last_error = saved;
  if (rc != SPARGE_OK) return 0;
  return sparge::lowbit_workspace_bytes(B, H, N, d, block_q);
}

}  // extern "C"

namespace {
// the low-bit branch, whole (phase kLowbitAll) or in its parts; arguments a
// part does not read may be null
int lowbit_impl(const char* what, int phase, const void* q, const void* k, const void* v,
                const int32_t* kv_idx, const int32_t* kv_cnt, int B, int H, int N, int d,
                int block_q, int block_k, float scale, void* o, void* workspace,
                size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_shape(B, H, N, d, block_q, block_k);
  if (rc != SPARGE_OK) return rc;
  const bool quant = phase == sparge::kLowbitAll, packs = phase != sparge::kLowbitAttend;
  const bool attends = phase != sparge::kLowbitPackV;
  if (!workspace || (quant && (!q || !k)) || (packs && !v) || (attends && (!o || !kv_idx || !kv_cnt)))
    return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if ((quant && (!aligned(q, 16) || !aligned(k, 16))) || (packs && !aligned(v, 16)) ||
      (attends && !aligned(o, 16)))
    return fail(SPARGE_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (attends && (!aligned(kv_idx, 4) || !aligned(kv_cnt, 4)))
    return fail(SPARGE_ERR_INVALID_ARG, "kv_idx and kv_cnt must be 4-byte aligned");
  if (attends && (!(scale > 0.0f) || !isfinite(scale)))
    return fail(SPARGE_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(workspace, 256)) return fail(SPARGE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < sparge::lowbit_workspace_bytes(B, H, N, d, block_q))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  sparge::LowbitLaunch a{};
  a.phase = phase;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = kv_idx;
  a.cnt = kv_cnt;
  a.o = static_cast<uint16_t*>(o);
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q;
  a.n_q = ceil_div(N, block_q);
  a.n_k = ceil_div(N, block_k);
  a.scale = scale;
  sparge::lowbit_layout(a, static_cast<unsigned char*>(workspace));
  const hipError_t e = sparge::launch_lowbit(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, what);
  return SPARGE_OK;
}
}  // namespace

extern "C" {

int sparge_attn_fwd_lowbit(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                           const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                           int block_k, float scale, void* o, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return lowbit_impl("sparge_attn_fwd_lowbit launch", sparge::kLowbitAll, q, k, v, kv_idx,
                     kv_cnt, B, H, N, d, block_q, block_k, scale, o, workspace,
                     workspace_bytes, stream);
}

int sparge_attn_lowbit_pack(const void* v, int B, int H, int N, int d, int block_q,
                            void* lowbit_workspace, size_t lowbit_workspace_bytes,
                            void* stream) {
  return lowbit_impl("sparge_attn_lowbit_pack launch", sparge::kLowbitPackV, nullptr, nullptr,
                     v, nullptr, nullptr, B, H, N, d, block_q, 64, 1.0f, nullptr,
                     lowbit_workspace, lowbit_workspace_bytes, stream);
}

int sparge_attn_fwd_lowbit_packed(const int32_t* kv_idx, const int32_t* kv_cnt, int B, int H,
                                  int N, int d, int block_q, int block_k, float scale, void* o,
                                  void* lowbit_workspace, size_t lowbit_workspace_bytes,
                                  void* stream) {
  return lowbit_impl("sparge_attn_fwd_lowbit_packed launch", sparge::kLowbitAttend, nullptr,
                     nullptr, nullptr, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o,
                     lowbit_workspace, lowbit_workspace_bytes, stream);
}

size_t svg2_attn_workspace_bytes(int B, int H, int N, int d, int block_q, int n_q_clusters,
                                 int n_k_clusters) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, block_q, 64);
  g_last_error = saved;
  if (rc != SPARGE_OK || n_q_clusters < 1 || n_k_clusters < 1 || n_q_clusters > N ||
      n_k_clusters > N || n_k_clusters > kMaxKeyBlocks)
    return 0;
  return sparge::svg2_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters);
}

}  // extern "C"

namespace {
int svg2_impl(int phase, const void* q, const void* k, const void* v, int B, int H, int N,
              int d, int block_q, int n_q_clusters, int n_k_clusters, int iters, float p_mass,
              float scale, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_shape(B, H, N, d, block_q, 64);
  if (rc != SPARGE_OK) return rc;
  const bool clusters = phase != sparge::kSvg2Attend, attends = phase != sparge::kSvg2Cluster;
  if ((clusters && (!q || !k || !v)) || (attends && !o) || !workspace)
    return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if ((clusters && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))) ||
      (attends && !aligned(o, 16)) || !aligned(workspace, 256))
    return fail(SPARGE_ERR_INVALID_ARG, "q, k, v, o must be 16-byte and workspace 256-byte aligned");
  if (n_q_clusters < 1 || n_k_clusters < 1 || n_q_clusters > N || n_k_clusters > N)
    return fail(SPARGE_ERR_INVALID_ARG, "cluster counts must lie in [1, N]");
  if (n_k_clusters > kMaxKeyBlocks)
    return fail(SPARGE_ERR_UNSUPPORTED, "at most 4096 key clusters");
  if (iters < 0 || iters > 1000) return fail(SPARGE_ERR_INVALID_ARG, "iters must lie in [0, 1000]");
  if (!(p_mass >= 0.0f) || !(scale > 0.0f) || !isfinite(scale))
    return fail(SPARGE_ERR_INVALID_ARG, "p_mass must be >= 0 and scale finite and > 0");
  if (workspace_bytes < sparge::svg2_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  sparge::Svg2Launch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q;
  a.Cq = n_q_clusters; a.Ck = n_k_clusters; a.iters = iters;
  a.scale = scale;
  a.p = (double)p_mass;
  a.phase = phase;
  sparge::svg2_layout(a, static_cast<unsigned char*>(workspace));
  const hipError_t e = sparge::launch_svg2(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "svg2_attn_fwd launch");
  return SPARGE_OK;
}
}  // namespace

extern "C" {

int svg2_attn_fwd(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                  int block_q, int n_q_clusters, int n_k_clusters, int iters, float p_mass,
                  float scale, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  return svg2_impl(sparge::kSvg2All, q, k, v, B, H, N, d, block_q, n_q_clusters, n_k_clusters,
                   iters, p_mass, scale, o, workspace, workspace_bytes, stream);
}

int svg2_attn_cluster(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                      int block_q, int n_q_clusters, int n_k_clusters, int iters, float p_mass,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return svg2_impl(sparge::kSvg2Cluster, q, k, v, B, H, N, d, block_q, n_q_clusters,
                   n_k_clusters, iters, p_mass, scale, nullptr, workspace, workspace_bytes,
                   stream);
}

int svg2_attn_apply(int B, int H, int N, int d, int block_q, int n_q_clusters, int n_k_clusters,
                    float scale, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  return svg2_impl(sparge::kSvg2Attend, nullptr, nullptr, nullptr, B, H, N, d, block_q,
                   n_q_clusters, n_k_clusters, 0, 0.0f, scale, o, workspace, workspace_bytes,
                   stream);
}

int svg2_attn_pair_counts(int B, int H, int N, int d, int block_q, int n_q_clusters,
                          int n_k_clusters, uint64_t* counts, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_shape(B, H, N, d, block_q, 64);
  if (rc != SPARGE_OK) return rc;
  if (!counts || !workspace) return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(counts, 8) || !aligned(workspace, 256))
    return fail(SPARGE_ERR_INVALID_ARG, "counts must be 8-byte and workspace 256-byte aligned");
  if (n_q_clusters < 1 || n_k_clusters < 1 || n_q_clusters > N || n_k_clusters > N)
    return fail(SPARGE_ERR_INVALID_ARG, "cluster counts must lie in [1, N]");
  if (n_k_clusters > kMaxKeyBlocks)
    return fail(SPARGE_ERR_UNSUPPORTED, "at most 4096 key clusters");
  if (workspace_bytes < sparge::svg2_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  sparge::Svg2Launch a{};
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q;
  a.Cq = n_q_clusters; a.Ck = n_k_clusters;
  sparge::svg2_layout(a, static_cast<unsigned char*>(workspace));
  const hipError_t e = sparge::launch_svg2_pairs(
      a, reinterpret_cast<unsigned long long*>(counts), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "svg2_attn_pair_counts launch");
  return SPARGE_OK;
}

size_t sparse_linear_bwd_workspace_bytes(int B, int H, int N, int d) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, d == 64 ? 64 : 128, 64);
  g_last_error = saved;
  if (rc != SPARGE_OK || ceil_div(N, 64) > kMaxKeyBlocks) return 0;
  return sparge::bwd_workspace_bytes(B, H, N, d, d, true);
}

int sparse_linear_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, const int32_t* kv_idx,
                           const int32_t* kv_cnt, const float* alpha, int B, int H, int N,
                           int d, int block_q, int block_k, float scale, float drop_below,
                           void* dq, void* dk, void* dv, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return bwd_impl("sparse_linear_attn_bwd launch", sparge::kLinAdd, q, k, v, o, d_o, lse, kv_idx,
                  kv_cnt, alpha, B, H, N, d, block_q, block_k, scale, drop_below, dq, dk, dv,
                  workspace, workspace_bytes, stream);
}

int sla2_mix_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* d_o, const float* lse, const int32_t* kv_idx,
                      const int32_t* kv_cnt, const float* alpha, int B, int H, int N, int d,
                      int block_q, int block_k, float scale, float drop_below, void* dq,
                      void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return bwd_impl("sla2_mix_attn_bwd launch", sparge::kLinMix, q, k, v, o, d_o, lse, kv_idx,
                  kv_cnt, alpha, B, H, N, d, block_q, block_k, scale, drop_below, dq, dk, dv,
                  workspace, workspace_bytes, stream);
}

int sparge_attn_pack(const void* v, int B, int H, int N, int d, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_shape(B, H, N, d, 128, 64);
  if (rc != SPARGE_OK) return rc;
  if (!v) return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(v, 16)) return fail(SPARGE_ERR_INVALID_ARG, "v must be 16-byte aligned");
  rc = check_attn_workspace(workspace, workspace_bytes, B, H, N, d);
  if (rc != SPARGE_OK) return rc;
  const sparge::AttnLaunch a =
      attn_args(nullptr, nullptr, v, nullptr, nullptr, B, H, N, d, 128, 64, 1.0f, nullptr,
                workspace);
  const hipError_t e = sparge::launch_attn(a, static_cast<hipStream_t>(stream), sparge::kPackOnly);
  if (e != hipSuccess) return hip_fail(e, "sparge_attn_pack launch");
  return SPARGE_OK;
}

int sparge_attn_fwd_packed(const void* q, const void* k, const int32_t* kv_idx,
                           const int32_t* kv_cnt, int B, int H, int N, int d, int block_q,
                           int block_k, float scale, void* o, const void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  // v is not read here; q stands in for it in the shared pointer checks
  int rc = check_attn_args(q, k, q, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o);
  if (rc == SPARGE_OK) rc = check_attn_workspace(workspace, workspace_bytes, B, H, N, d);
  if (rc != SPARGE_OK) return rc;
  const sparge::AttnLaunch a = attn_args(q, k, nullptr, kv_idx, kv_cnt, B, H, N, d, block_q,
                                         block_k, scale, o, const_cast<void*>(workspace));
  const hipError_t e =
      sparge::launch_attn(a, static_cast<hipStream_t>(stream), sparge::kAttendOnly);
  if (e != hipSuccess) return hip_fail(e, "sparge_attn_fwd_packed launch");
  return SPARGE_OK;
}

size_t sparse_linear_workspace_bytes(int B, int H, int N, int d) {
  const std::string saved = g_last_error;
  const int rc = check_shape(B, H, N, d, 128, 64);
  g_last_error = saved;
  if (rc != SPARGE_OK || ceil_div(N, 64) > sparge::kLinMaxKeyBlocks) return 0;
  return sparge::linear_workspace_bytes(B, H, N, d, d);
}

}  // extern "C"

namespace {

int linear_impl(const char* name, int mode, const void* q, const void* k, const void* v,
                const int32_t* kv_idx, const int32_t* kv_cnt, const float* alpha, int B, int H,
                int N, int d, int block_q, int block_k, float scale, float drop_below, void* o,
                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_attn_args(q, k, v, kv_idx, kv_cnt, B, H, N, d, block_q, block_k, scale, o);
  if (rc != SPARGE_OK) return rc;
  if (!alpha || !workspace) return fail(SPARGE_ERR_INVALID_ARG, "null pointer argument");
  // the mix reads alpha[h][4c .. 4c+3] as one 16-byte load
  if (!aligned(alpha, mode == sparge::kLinMix ? 16 : 4) || !aligned(workspace, 16) ||
      !aligned(lse, 4))
    return fail(SPARGE_ERR_INVALID_ARG, "alpha / workspace / lse misaligned");
  if (block_q != d)
    return fail(SPARGE_ERR_UNSUPPORTED, "the linear branch is built for block_q == d (64 or 128)");
  if (ceil_div(N, block_k) > sparge::kLinMaxKeyBlocks)
    return fail(SPARGE_ERR_UNSUPPORTED, "the linear branch supports at most 4096 key blocks");
  if (workspace_bytes < sparge::linear_workspace_bytes(B, H, N, d, block_q))
    return fail(SPARGE_ERR_INVALID_ARG, "workspace too small");
  sparge::AttnLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = kv_idx;
  a.cnt = kv_cnt;
  a.o = static_cast<uint16_t*>(o);
  a.B = B; a.H = H; a.N = N; a.d = d; a.block_q = block_q;
  a.n_q = ceil_div(N, block_q);
  a.n_k = ceil_div(N, block_k);
  a.scale = scale;
  a.alpha = alpha;
  a.lin_mode = mode;
  a.drop_below = drop_below;
  a.lse = lse;
  sparge::linear_layout(a, static_cast<unsigned char*>(workspace), B, H, N, d, block_q);
  const hipError_t e = sparge::launch_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, name);
  return SPARGE_OK;
}

}  // namespace

extern "C" {

int sparse_linear_attn_fwd(const void* q, const void* k, const void* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, const float* alpha,
                           int B, int H, int N, int d, int block_q, int block_k, float scale,
                           float drop_below, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return linear_impl("sparse_linear_attn_fwd launch", sparge::kLinAdd, q, k, v, kv_idx, kv_cnt,
                     alpha, B, H, N, d, block_q, block_k, scale, drop_below, o, lse, workspace,
                     workspace_bytes, stream);
}

int sla2_mix_attn_fwd(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                      const int32_t* kv_cnt, const float* alpha, int B, int H, int N, int d,
                      int block_q, int block_k, float scale, float drop_below, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl("sla2_mix_attn_fwd launch", sparge::kLinMix, q, k, v, kv_idx, kv_cnt,
                     alpha, B, H, N, d, block_q, block_k, scale, drop_below, o, lse, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"
