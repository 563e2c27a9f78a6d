// C-ABI front end: argument validation, kernel choice, launch, error state.
//
// Follows the execution flow of "Using cuDNN in Python" (tensor descriptors
// with dims + strides, a support check before execution, execute(pointers,
// workspace) on a stream, caller-side synchronisation) and the error
// reporting of the cuDNN 9 blog ("Improved error reporting": specific codes
// plus a programmatic last-error string). Unsupported problems are reported,
// never silently run on another path (the JAX attention codelab's step 6:
// forcing a backend raises instead of falling back).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "sdpa.h"
#include "sdpa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local sdpa::TimingEvents g_timing{};

int log_level() {
  static int level = [] {
    const char* s = getenv("SDPA_LOG_LEVEL");
    return s ? atoi(s) : 0;
  }();
  return level;
}

sdpa_status_t fail(sdpa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (log_level() >= 1) fprintf(stderr, "[sdpa] %s: %s\n", sdpa_status_string(st), buf);
  return st;
}

int elem_bytes(sdpa_dtype_t t) {
  switch (t) {
    case SDPA_F32: return 4;
    case SDPA_F16:
    case SDPA_BF16: return 2;
    case SDPA_FP8_E4M3:
    case SDPA_FP8_E5M2: return 1;
  }
  return 0;
}

bool valid_dtype(int t) { return t >= SDPA_F32 && t <= SDPA_FP8_E5M2; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Checks one tensor's pointer and strides. Returns SDPA_OK or an error.
sdpa_status_t check_tensor(const char* name, const void* p, const int64_t* st, int eb,
                           sdpa::Strides3* out) {
  if (p == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (st == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "%s stride array is NULL", name);
  if (st[3] != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "%s d-stride is %lld, must be 1", name, (long long)st[3]);
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "%s stride[%d] is negative", name, i);
  if (((uintptr_t)p) % 16 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "%s is not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i)
    if ((st[i] * eb) % 16 != 0)
      return fail(SDPA_ERR_NOT_SUPPORTED, "%s stride[%d]=%lld is not a multiple of 16 bytes", name, i,
                  (long long)st[i]);
  out->b = st[0];
  out->h = st[1];
  out->s = st[2];
  return SDPA_OK;
}

sdpa_status_t check_mask(sdpa_mask_t mask, const int32_t* seq_len_q, const int32_t* seq_len_kv) {
  if (mask != SDPA_MASK_NONE && mask != SDPA_MASK_CAUSAL && mask != SDPA_MASK_CAUSAL_BOTTOM_RIGHT)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "mask must be SDPA_MASK_NONE, _CAUSAL or _CAUSAL_BOTTOM_RIGHT (got %d)",
                (int)mask);
  if ((((uintptr_t)seq_len_q) | ((uintptr_t)seq_len_kv)) % 4 != 0)
    return fail(SDPA_ERR_NOT_SUPPORTED, "seq_len arrays must be 4-byte aligned");
  return SDPA_OK;
}

// Validates the score modifiers and converts them; io is the input dtype.
sdpa_status_t check_mod(const sdpa_score_mod_t* mod, sdpa_dtype_t io, sdpa::ScoreMod* out) {
  *out = sdpa::ScoreMod{};
  out->drop_k8 = 256;  // no dropout
  out->drop_scale = 1.f;
  if (mod == nullptr) return SDPA_OK;
  if (!(mod->dropout_p >= 0.f && mod->dropout_p <= 1.f))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "dropout_p must be in [0, 1]");
  if (mod->alibi_slopes == nullptr && mod->bias == nullptr && mod->dropout_p == 0.f) return SDPA_OK;
  if (io == SDPA_FP8_E4M3) return fail(SDPA_ERR_NOT_SUPPORTED, "score modifiers are not supported with fp8 inputs");
  if (((uintptr_t)mod->alibi_slopes) % 4 != 0)
    return fail(SDPA_ERR_NOT_SUPPORTED, "alibi_slopes must be 4-byte aligned");
  out->slopes = mod->alibi_slopes;
  if (mod->bias != nullptr) {
    if (!(mod->bias_dtype == SDPA_F32 || (mod->bias_dtype == io && io != SDPA_F32)))
      return fail(SDPA_ERR_NOT_SUPPORTED, "bias dtype %d must be F32 or the io dtype", (int)mod->bias_dtype);
    const int eb = mod->bias_dtype == SDPA_F32 ? 4 : 2;
    if (mod->bias_stride[3] != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "bias s_kv stride must be 1");
    if (((uintptr_t)mod->bias) % 16 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "bias is not 16-byte aligned");
    for (int i = 0; i < 3; ++i)
      if (mod->bias_stride[i] < 0 || (mod->bias_stride[i] * eb) % 16 != 0)
        return fail(SDPA_ERR_NOT_SUPPORTED, "bias stride %d (%lld) must be >= 0 and a multiple of 16 bytes", i,
                    (long long)mod->bias_stride[i]);
    out->bias = mod->bias;
    out->bias_f32 = eb == 4;
    out->bb = mod->bias_stride[0];
    out->bh = mod->bias_stride[1];
    out->bs = mod->bias_stride[2];
  }
  if (mod->dropout_p > 0.f) {
    if (io != SDPA_BF16 && io != SDPA_F16)
      return fail(SDPA_ERR_NOT_SUPPORTED, "dropout needs BF16 or F16 inputs");
    // keep iff random byte < k8 = round((1 - p) * 256), ties to even; kept weights scale by 256 / k8
    out->drop_k8 = (int)nearbyint((1.0 - (double)mod->dropout_p) * 256.0);
    out->drop_scale = out->drop_k8 > 0 ? (float)(256.0 / out->drop_k8) : 0.f;
    out->seed_lo = (uint32_t)(mod->dropout_seed & 0xFFFFFFFFu);
    out->seed_hi = (uint32_t)(mod->dropout_seed >> 32);
    out->offset = mod->dropout_offset;
  }
  return SDPA_OK;
}

sdpa_status_t check_sizes(int b, int h_q, int h_kv, int s_q, int s_kv, int d) {
  if (b < 0 || s_q < 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "b=%d and s_q=%d must be >= 0", b, s_q);
  if (h_q < 1 || h_kv < 1 || s_kv < 1 || d < 1)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "h_q=%d, h_kv=%d, s_kv=%d, d=%d must be >= 1", h_q, h_kv, s_kv, d);
  if (h_q % h_kv != 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  // grid size: query blocks x b x h_q must fit a 32-bit grid
  if ((int64_t)((s_q + 31) / 32) * b * h_q > 0x7fffffffLL)
    return fail(SDPA_ERR_NOT_SUPPORTED, "problem too large for one launch");
  return SDPA_OK;
}

sdpa_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SDPA_OK;
}

// Scratch of sdpa_fwd_noalloc: the split-KV forward's per-split partials,
// in a file-scope device array so that the entry point allocates nothing.
// Each GPU the library runs on holds its own copy until the process ends. In
// host code `scratch` is only a stand-in for the symbol, not a device address:
// every use goes through scratch_on(), which resolves the address per device
// with hipGetSymbolAddress (with that device current) and keeps it.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or null with the
// error recorded.
void* scratch_on(sdpa_status_t* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(SDPA_ERR_NOT_SUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, kMaxDevices - 1);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *st = e != hipSuccess ? hip_status(e, "hipGetSymbolAddress(scratch)")
                            : fail(SDPA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *st = SDPA_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* sdpa_status_string(sdpa_status_t s) {
  switch (s) {
    case SDPA_OK: return "SDPA_OK";
    case SDPA_ERR_INVALID_ARGUMENT: return "SDPA_ERR_INVALID_ARGUMENT";
    case SDPA_ERR_NOT_SUPPORTED: return "SDPA_ERR_NOT_SUPPORTED";
    case SDPA_ERR_WORKSPACE_TOO_SMALL: return "SDPA_ERR_WORKSPACE_TOO_SMALL";
    case SDPA_ERR_HIP: return "SDPA_ERR_HIP";
  }
  return "SDPA_ERR_UNKNOWN";
}

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

sdpa_status_t sdpa_mfma_probe(sdpa_dtype_t dtype, int blocks, int iters, uint64_t* stamps, hipStream_t stream) {
  g_last_error.clear();
  if (dtype != SDPA_BF16 && dtype != SDPA_FP8_E4M3)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "mfma probe: dtype must be BF16 or FP8_E4M3 (got %d)", (int)dtype);
  if (blocks < 1 || iters < 1)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "mfma probe: blocks=%d and iters=%d must be >= 1", blocks, iters);
  if (stamps == nullptr || ((uintptr_t)stamps) % 16 != 0)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "mfma probe: stamps must be a non-NULL 16-byte aligned device pointer");
  return hip_status(sdpa::launch_mfma_probe(dtype == SDPA_FP8_E4M3, blocks, iters, stamps, stream), "probe launch");
}

sdpa_status_t sdpa_alibi_slopes(int h_q, float* slopes_host) {
  g_last_error.clear();
  if (h_q < 1 || slopes_host == nullptr)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "alibi slopes: h_q=%d must be >= 1 and the output non-NULL", h_q);
  int n = 1;  // largest power of two <= h_q
  while (2 * n <= h_q) n *= 2;
  // Geometric sequence of n heads: slope i = 2^(-8 (i + 1) / n).
  for (int i = 0; i < n; ++i) slopes_host[i] = (float)exp2(-8.0 * (i + 1) / n);
  // The remaining heads take the even-indexed slopes of the 2n-head sequence,
  // 2^(-8 (2 k + 1) / (2 n)), k = 0, 1, ...
  for (int k = 0; n + k < h_q; ++k) slopes_host[n + k] = (float)exp2(-8.0 * (2 * k + 1) / (2.0 * n));
  return SDPA_OK;
}

sdpa_status_t sdpa_set_timing_events(hipEvent_t* events, int n) {
  g_last_error.clear();
  if (n < 0 || n > 8 || (n > 0 && events == nullptr))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "timing events: n=%d must be in [0, 8] with a non-NULL array", n);
  g_timing.n = events == nullptr ? 0 : n;
  for (int i = 0; i < g_timing.n; ++i) g_timing.ev[i] = events[i];
  return SDPA_OK;
}

sdpa_status_t sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int b, int h_q,
                       int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                       const int64_t k_stride[4], const int64_t v_stride[4], const int64_t o_stride[4],
                       float attn_scale, int causal, sdpa_dtype_t in_dtype, sdpa_dtype_t out_dtype,
                       const sdpa_fp8_scales_t* fp8, hipStream_t stream) {
  g_last_error.clear();
  if (causal != 0 && causal != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  return sdpa_fwd_ex(q, k, v, o, lse, b, h_q, h_kv, s_q, s_kv, d, q_stride, k_stride, v_stride, o_stride,
                     attn_scale, causal ? SDPA_MASK_CAUSAL : SDPA_MASK_NONE, nullptr, nullptr, nullptr, in_dtype,
                     out_dtype, fp8, nullptr, 0, stream);
}

size_t sdpa_fwd_workspace_size(int b, int h_q, int h_kv, int s_q, int s_kv, int d, sdpa_dtype_t in_dtype) {
  if (b <= 0 || h_q <= 0 || h_kv <= 0 || s_q <= 0 || s_kv <= 0 || d <= 0 || h_q % h_kv != 0) return 0;
  if (in_dtype != SDPA_BF16 && in_dtype != SDPA_F16) return 0;
  const sdpa::Io io = in_dtype == SDPA_BF16 ? sdpa::Io::BF16 : sdpa::Io::F16;
  return sdpa::plan_decode(b, h_q, h_kv, s_q, s_kv, d, io).ws_bytes;
}

}  // extern "C"

namespace {

// The forward behind sdpa_fwd_ex and sdpa_fwd_noalloc. With static_scratch the
// split-KV path takes its partials from the device's static scratch array
// (the workspace arguments are unused); otherwise from the caller's workspace.
sdpa_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int b, int h_q, int h_kv,
                       int s_q, int s_kv, int d, const int64_t q_stride[4], const int64_t k_stride[4],
                       const int64_t v_stride[4], const int64_t o_stride[4], float attn_scale, sdpa_mask_t mask,
                       const int32_t* seq_len_q, const int32_t* seq_len_kv, const sdpa_score_mod_t* mod,
                       sdpa_dtype_t in_dtype, sdpa_dtype_t out_dtype, const sdpa_fp8_scales_t* fp8,
                       void* workspace, size_t workspace_bytes, bool static_scratch, hipStream_t stream) {
  sdpa_status_t st;
  if ((st = check_sizes(b, h_q, h_kv, s_q, s_kv, d)) != SDPA_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype (%d, %d)", (int)in_dtype, (int)out_dtype);
  if ((st = check_mask(mask, seq_len_q, seq_len_kv)) != SDPA_OK) return st;
  if (!(attn_scale > 0.f) || !isfinite(attn_scale))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_scale must be finite and > 0");
  if ((in_dtype == SDPA_FP8_E4M3) != (fp8 != nullptr))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "fp8 scales must be given iff in_dtype is FP8_E4M3");
  if (fp8 != nullptr) {
    const float f[5] = {fp8->descale_q, fp8->descale_k, fp8->descale_v, fp8->scale_p, fp8->descale_p};
    for (float x : f)
      if (!(x > 0.f) || !isfinite(x)) return fail(SDPA_ERR_INVALID_ARGUMENT, "fp8 factors must be finite and > 0");
    if (fp8->scale_p > 448.f)
      return fail(SDPA_ERR_INVALID_ARGUMENT, "fp8 scale_p must be <= 448 (P <= 1 is quantised as P * scale_p)");
  }
  sdpa::Io io;
  bool ok = false;
  if (in_dtype == SDPA_F32 && out_dtype == SDPA_F32) {
    io = sdpa::Io::F32;
    ok = d == 64 || d == 128;
  } else if (in_dtype == SDPA_F16 && out_dtype == SDPA_F16) {
    io = sdpa::Io::F16;
    ok = d == 64 || d == 128;
  } else if (in_dtype == SDPA_BF16 && out_dtype == SDPA_BF16) {
    io = sdpa::Io::BF16;
    ok = d == 64 || d == 128;
  } else if (in_dtype == SDPA_FP8_E4M3 && out_dtype == SDPA_BF16) {
    io = sdpa::Io::FP8;
    ok = d == 128 || d == 256;
  }
  if (!ok)
    return fail(SDPA_ERR_NOT_SUPPORTED, "no forward kernel for in=%d out=%d d=%d", (int)in_dtype, (int)out_dtype, d);

  sdpa::FwdArgs a{};
  if ((st = check_mod(mod, in_dtype, &a.mod)) != SDPA_OK) return st;
  // Empty problem: nothing to compute or write; the (possibly NULL) pointers of
  // empty tensors are not inspected.
  if (b == 0 || s_q == 0) return SDPA_OK;
  const int ein = elem_bytes(in_dtype), eout = elem_bytes(out_dtype);
  if ((st = check_tensor("q", q, q_stride, ein, &a.qs)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, ein, &a.ks)) != SDPA_OK) return st;
  if ((st = check_tensor("v", v, v_stride, ein, &a.vs)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, eout, &a.os)) != SDPA_OK) return st;
  if (lse != nullptr && ((uintptr_t)lse) % 4 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "lse is not 4-byte aligned");

  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.b = b;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.s_q = s_q;
  a.s_kv = s_kv;
  a.d = d;
  a.causal = mask != SDPA_MASK_NONE;
  a.bottom_right = mask == SDPA_MASK_CAUSAL_BOTTOM_RIGHT;
  a.seq_q = seq_len_q;
  a.seq_kv = seq_len_kv;
  a.scale = attn_scale;
  if (fp8 != nullptr) {
    a.scale = attn_scale * fp8->descale_q * fp8->descale_k;
    a.descale_v = fp8->descale_v;
    a.scale_p = fp8->scale_p;
    a.descale_p = fp8->descale_p;
  }
  if (log_level() >= 2)
    fprintf(stderr, "[sdpa] fwd io=%d d=%d b=%d h_q=%d h_kv=%d s_q=%d s_kv=%d mask=%d lens=%d\n", (int)io, d, b,
            h_q, h_kv, s_q, s_kv, (int)mask, (seq_len_q != nullptr) + 2 * (seq_len_kv != nullptr));
  // Few query rows against many keys: the split-KV path, when its workspace
  // (if it needs one) is given; otherwise the row-block kernel.
  const sdpa::DecodePlan plan = sdpa::plan_decode(b, h_q, h_kv, s_q, s_kv, d, io);
  if (static_scratch && plan.use && !sdpa::has_mod(a.mod) && plan.ws_bytes > 0) {
    if (plan.ws_bytes > kScratchBytes)
      return fail(SDPA_ERR_NOT_SUPPORTED,
                  "the split-KV forward needs %zu bytes of scratch; the static scratch of sdpa_fwd_noalloc holds %zu",
                  plan.ws_bytes, kScratchBytes);
    if ((workspace = scratch_on(&st)) == nullptr) return st;
    workspace_bytes = kScratchBytes;
  }
  const bool split_kv = plan.use && !sdpa::has_mod(a.mod) && (plan.ws_bytes == 0 || workspace != nullptr);
  if (split_kv && plan.ws_bytes > 0) {
    if (workspace_bytes < plan.ws_bytes)
      return fail(SDPA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the split-KV forward needs %zu",
                  workspace_bytes, plan.ws_bytes);
    if (((uintptr_t)workspace) % 16 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "workspace is not 16-byte aligned");
  }
  if (log_level() >= 2 && split_kv)
    fprintf(stderr, "[sdpa] fwd split-KV: n_split=%d split_keys=%d row_blocks=%d\n", plan.n_split,
            plan.split_keys, plan.n_rb);
  if (g_timing.n >= 2) (void)hipEventRecord(g_timing.ev[0], stream);
  hipError_t e;
  if (split_kv) {
    e = sdpa::launch_fwd_decode(a, plan, workspace, io, stream);
  } else {
    switch (io) {
      case sdpa::Io::F32: e = sdpa::launch_fwd_f32(a, stream); break;
      case sdpa::Io::FP8: e = sdpa::launch_fwd_fp8(a, stream); break;
      default: e = sdpa::launch_fwd_mfma(a, io, stream); break;
    }
  }
  if (e == hipSuccess && g_timing.n >= 2) e = hipEventRecord(g_timing.ev[1], stream);
  return hip_status(e, "forward launch");
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int b, int h_q,
                          int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                          const int64_t k_stride[4], const int64_t v_stride[4], const int64_t o_stride[4],
                          float attn_scale, sdpa_mask_t mask, const int32_t* seq_len_q,
                          const int32_t* seq_len_kv, const sdpa_score_mod_t* mod, sdpa_dtype_t in_dtype,
                          sdpa_dtype_t out_dtype, const sdpa_fp8_scales_t* fp8, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  return fwd_impl(q, k, v, o, lse, b, h_q, h_kv, s_q, s_kv, d, q_stride, k_stride, v_stride, o_stride, attn_scale,
                  mask, seq_len_q, seq_len_kv, mod, in_dtype, out_dtype, fp8, workspace, workspace_bytes, false,
                  stream);
}

sdpa_status_t sdpa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int b, int h_q,
                               int h_kv, int s_q, int s_kv, int d, const int64_t q_stride[4],
                               const int64_t k_stride[4], const int64_t v_stride[4], const int64_t o_stride[4],
                               float attn_scale, sdpa_mask_t mask, const int32_t* seq_len_q,
                               const int32_t* seq_len_kv, const sdpa_score_mod_t* mod, sdpa_dtype_t in_dtype,
                               sdpa_dtype_t out_dtype, const sdpa_fp8_scales_t* fp8, hipStream_t stream) {
  g_last_error.clear();
  return fwd_impl(q, k, v, o, lse, b, h_q, h_kv, s_q, s_kv, d, q_stride, k_stride, v_stride, o_stride, attn_scale,
                  mask, seq_len_q, seq_len_kv, mod, in_dtype, out_dtype, fp8, nullptr, 0, true, stream);
}

size_t sdpa_bwd_workspace_size(int b, int h_q, int h_kv, int s_q, int s_kv, int d, int causal,
                               sdpa_dtype_t dtype) {
  (void)causal;
  if (b <= 0 || h_q <= 0 || h_kv <= 0 || s_q <= 0 || s_kv <= 0 || d <= 0) return 0;
  (void)dtype;  // the fp8 backward needs the same D and partial buffers
  return sdpa::bwd_workspace_bytes(b, h_q, h_kv, s_q, s_kv, d);
}

sdpa_status_t sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int b, int h_q, int h_kv, int s_q,
                       int s_kv, int d, const int64_t q_stride[4], const int64_t k_stride[4],
                       const int64_t v_stride[4], const int64_t o_stride[4], const int64_t do_stride[4],
                       const int64_t dq_stride[4], const int64_t dk_stride[4], const int64_t dv_stride[4],
                       float attn_scale, int causal, sdpa_dtype_t dtype, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (causal != 0 && causal != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  return sdpa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, b, h_q, h_kv, s_q, s_kv, d, q_stride, k_stride,
                     v_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride, attn_scale,
                     causal ? SDPA_MASK_CAUSAL : SDPA_MASK_NONE, nullptr, nullptr, nullptr, dtype, workspace,
                     workspace_bytes, stream);
}

sdpa_status_t sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, int b, int h_q, int h_kv, int s_q,
                          int s_kv, int d, const int64_t q_stride[4], const int64_t k_stride[4],
                          const int64_t v_stride[4], const int64_t o_stride[4], const int64_t do_stride[4],
                          const int64_t dq_stride[4], const int64_t dk_stride[4], const int64_t dv_stride[4],
                          float attn_scale, sdpa_mask_t mask, const int32_t* seq_len_q,
                          const int32_t* seq_len_kv, const sdpa_score_mod_t* mod, sdpa_dtype_t dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  sdpa_status_t st;
  if ((st = check_sizes(b, h_q, h_kv, s_q, s_kv, d)) != SDPA_OK) return st;
  if (!valid_dtype(dtype)) return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if ((st = check_mask(mask, seq_len_q, seq_len_kv)) != SDPA_OK) return st;
  if (!(attn_scale > 0.f) || !isfinite(attn_scale))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_scale must be finite and > 0");
  if (!((dtype == SDPA_BF16 || dtype == SDPA_F16) && (d == 64 || d == 128)))
    return fail(SDPA_ERR_NOT_SUPPORTED, "no backward kernel for dtype=%d d=%d", (int)dtype, d);
  sdpa::BwdArgs a{};
  if ((st = check_mod(mod, dtype, &a.mod)) != SDPA_OK) return st;
  const int eb = elem_bytes(dtype);
  const sdpa::Io io = dtype == SDPA_BF16 ? sdpa::Io::BF16 : sdpa::Io::F16;
  if (b == 0) return SDPA_OK;  // empty problem: every tensor is empty
  if (s_q == 0) {
    // No query rows: dK = dV = 0; only those two tensors are touched.
    if ((st = check_tensor("dk", dk, dk_stride, eb, &a.dks)) != SDPA_OK) return st;
    if ((st = check_tensor("dv", dv, dv_stride, eb, &a.dvs)) != SDPA_OK) return st;
    a.dk = dk;
    a.dv = dv;
    a.b = b;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.s_kv = s_kv;
    a.d = d;
    return hip_status(sdpa::launch_zero_dkdv(a, io, stream), "zero dK/dV launch");
  }
  if (lse == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse is required by the backward");
  if ((st = check_tensor("q", q, q_stride, eb, &a.qs)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, eb, &a.ks)) != SDPA_OK) return st;
  if ((st = check_tensor("v", v, v_stride, eb, &a.vs)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, eb, &a.os)) != SDPA_OK) return st;
  if ((st = check_tensor("dout", dout, do_stride, eb, &a.dos)) != SDPA_OK) return st;
  if ((st = check_tensor("dq", dq, dq_stride, eb, &a.dqs)) != SDPA_OK) return st;
  if ((st = check_tensor("dk", dk, dk_stride, eb, &a.dks)) != SDPA_OK) return st;
  if ((st = check_tensor("dv", dv, dv_stride, eb, &a.dvs)) != SDPA_OK) return st;
  if (((uintptr_t)lse) % 4 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "lse is not 4-byte aligned");
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.b = b;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.s_q = s_q;
  a.s_kv = s_kv;
  a.d = d;
  a.causal = mask != SDPA_MASK_NONE;
  a.bottom_right = mask == SDPA_MASK_CAUSAL_BOTTOM_RIGHT;
  a.seq_q = seq_len_q;
  a.seq_kv = seq_len_kv;
  a.scale = attn_scale;
  a.dq_scale = attn_scale;
  a.dk_scale = attn_scale;
  a.dv_scale = 1.f;
  a.delta_scale = 1.f;
  const size_t need = sdpa::bwd_workspace_bytes(b, h_q, h_kv, s_q, s_kv, d);
  if (workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (workspace == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)workspace) % 16 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "workspace is not 16-byte aligned");
  a.delta = (float*)workspace;
  if (log_level() >= 2)
    fprintf(stderr, "[sdpa] bwd io=%d d=%d b=%d h_q=%d h_kv=%d s_q=%d s_kv=%d mask=%d lens=%d\n", (int)io, d, b,
            h_q, h_kv, s_q, s_kv, (int)mask, (seq_len_q != nullptr) + 2 * (seq_len_kv != nullptr));
  return hip_status(sdpa::launch_bwd(a, io, stream, g_timing), "backward launch");
}

// The fp8 backward (JAX attention codelab, step 10, HYBRID format). With
// codes Qc, Kc, Vc, dOc and descales sq, sk, sv, so (real X = Xc * sX), and
// the kernels' quantised Pc = e4m3(P * sp), dSc = fp8(dS * sds):
//   S  = attn_scale * sq * sk * Qc Kc^T      (softmax scale)
//   dP = so * sv * dOc Vc^T,  D = so * rowsum(dOc * O),  dS = P * (dP - D)
//   dQ = attn_scale * dS K   = (attn_scale * sk / sds) * dSc Kc
//   dK = attn_scale * dS^T Q = (attn_scale * sq / sds) * dSc^T Qc
//   dV = P^T dO              = (so / sp) * Pc^T dOc
sdpa_status_t sdpa_bwd_fp8(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int b, int h_q, int h_kv, int s_q,
                           int s_kv, int d, const int64_t q_stride[4], const int64_t k_stride[4],
                           const int64_t v_stride[4], const int64_t o_stride[4], const int64_t do_stride[4],
                           const int64_t dq_stride[4], const int64_t dk_stride[4], const int64_t dv_stride[4],
                           float attn_scale, sdpa_mask_t mask, const int32_t* seq_len_q, const int32_t* seq_len_kv,
                           sdpa_dtype_t do_dtype, const sdpa_fp8_bwd_scales_t* scales, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  sdpa_status_t st;
  if ((st = check_sizes(b, h_q, h_kv, s_q, s_kv, d)) != SDPA_OK) return st;
  if ((st = check_mask(mask, seq_len_q, seq_len_kv)) != SDPA_OK) return st;
  if (!(attn_scale > 0.f) || !isfinite(attn_scale))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_scale must be finite and > 0");
  if (do_dtype != SDPA_FP8_E5M2 && do_dtype != SDPA_FP8_E4M3)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "do_dtype must be FP8_E5M2 or FP8_E4M3 (got %d)", (int)do_dtype);
  if (scales == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "fp8 scale factors are NULL");
  const float sq = scales->descale_q, sk = scales->descale_k, sv = scales->descale_v, so = scales->descale_do;
  for (float x : {sq, sk, sv, so})
    if (!(x > 0.f) || !isfinite(x)) return fail(SDPA_ERR_INVALID_ARGUMENT, "fp8 descale factors must be finite and > 0");
  const float sp = scales->scale_p, sds = scales->scale_ds;
  if (!(sp > 0.f) || !(sp <= 448.f))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "scale_p must be in (0, 448] (P * scale_p must fit e4m3), got %g", sp);
  if (!(sds > 0.f) || !isfinite(sds)) return fail(SDPA_ERR_INVALID_ARGUMENT, "scale_ds must be finite and > 0");
  if (scales->ds_dtype != SDPA_FP8_E4M3 && scales->ds_dtype != SDPA_FP8_E5M2)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "ds_dtype must be FP8_E4M3 or FP8_E5M2 (got %d)", (int)scales->ds_dtype);
  if (((uintptr_t)scales->amax_ds) % 4 != 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "amax_ds is not 4-byte aligned");
  if (!(d == 64 || d == 128)) return fail(SDPA_ERR_NOT_SUPPORTED, "no fp8 backward for d=%d", d);
  sdpa::BwdArgs a{};
  a.mod.drop_k8 = 256;  // no score modifiers
  a.mod.drop_scale = 1.f;
  if (b == 0) return SDPA_OK;
  if (s_q == 0) {
    if ((st = check_tensor("dk", dk, dk_stride, 2, &a.dks)) != SDPA_OK) return st;
    if ((st = check_tensor("dv", dv, dv_stride, 2, &a.dvs)) != SDPA_OK) return st;
    a.dk = dk;
    a.dv = dv;
    a.b = b;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.s_kv = s_kv;
    a.d = d;
    return hip_status(sdpa::launch_zero_dkdv(a, sdpa::Io::BF16, stream), "zero dK/dV launch");
  }
  if (lse == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse is required by the backward");
  if ((st = check_tensor("q", q, q_stride, 1, &a.qs)) != SDPA_OK) return st;
  if ((st = check_tensor("k", k, k_stride, 1, &a.ks)) != SDPA_OK) return st;
  if ((st = check_tensor("v", v, v_stride, 1, &a.vs)) != SDPA_OK) return st;
  if ((st = check_tensor("dout", dout, do_stride, 1, &a.dos)) != SDPA_OK) return st;
  if ((st = check_tensor("o", o, o_stride, 2, &a.os)) != SDPA_OK) return st;
  if ((st = check_tensor("dq", dq, dq_stride, 2, &a.dqs)) != SDPA_OK) return st;
  if ((st = check_tensor("dk", dk, dk_stride, 2, &a.dks)) != SDPA_OK) return st;
  if ((st = check_tensor("dv", dv, dv_stride, 2, &a.dvs)) != SDPA_OK) return st;
  if (((uintptr_t)lse) % 4 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "lse is not 4-byte aligned");
  const size_t need = sdpa::bwd_workspace_bytes(b, h_q, h_kv, s_q, s_kv, d);
  if (workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (workspace == nullptr) return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)workspace) % 16 != 0) return fail(SDPA_ERR_NOT_SUPPORTED, "workspace is not 16-byte aligned");
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.b = b;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.s_q = s_q;
  a.s_kv = s_kv;
  a.d = d;
  a.causal = mask != SDPA_MASK_NONE;
  a.bottom_right = mask == SDPA_MASK_CAUSAL_BOTTOM_RIGHT;
  a.seq_q = seq_len_q;
  a.seq_kv = seq_len_kv;
  // Real values: Q = q * sq, K = k * sk, V = v * sv, dO = do * so, P = p8 / sp,
  // dS = ds8 / sds; each product's factors multiply its fp32 accumulator.
  a.scale = attn_scale * sq * sk;
  a.dq_scale = attn_scale * sk / sds;
  a.dk_scale = attn_scale * sq / sds;
  a.dv_scale = so / sp;
  a.delta_scale = so;
  a.delta = (float*)workspace;
  a.f8.dp_scale = so * sv;
  a.f8.scale_p = sp;
  a.f8.scale_ds = sds;
  a.f8.amax_ds = scales->amax_ds;
  a.f8.do_e5m2 = do_dtype == SDPA_FP8_E5M2;
  a.f8.ds_e5m2 = scales->ds_dtype == SDPA_FP8_E5M2;
  if (log_level() >= 2)
    fprintf(stderr, "[sdpa] bwd_fp8 d=%d b=%d h_q=%d h_kv=%d s_q=%d s_kv=%d mask=%d do=%d ds=%d\n", d, b, h_q, h_kv,
            s_q, s_kv, (int)mask, (int)do_dtype, (int)scales->ds_dtype);
  return hip_status(sdpa::launch_bwd_fp8(a, stream, g_timing), "fp8 backward launch");
}

}  // extern "C"
