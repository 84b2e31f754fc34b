// C ABI of the MoE FFN library: argument checks, error reporting, workspace
// carving and path selection.  Every check runs before anything is enqueued;
// errors name the parameter and its value and never fall back silently to
// another path (yfxerp.com static review §5.2 "explicit error path" and §6.2
// "messages carry the parameter name and current value").
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "strata_moe.h"
#include "moe_internal.h"

using namespace strata;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fn, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(fn) + ": " + buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return STRATA_OK;
}

int hip_fail(const char *fn, hipError_t e) {
  return fail(STRATA_ERR_HIP, fn, "HIP error %d (%s)", (int)e, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(fn, p)                                                                      \
  do {                                                                                          \
    if ((p) == nullptr) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "%s is NULL", #p);        \
    if (!aligned16(p))                                                                          \
      return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "%s=%p is not 16-byte aligned", #p, (const void *)(p)); \
  } while (0)

// Common T/E/k checks.
int check_tek(const char *fn, long long T, long long E, long long k) {
  if (T < 0) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "T=%lld is negative", T);
  if (E < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "E=%lld must be >= 1", E);
  if (E > kMaxExperts) return fail(STRATA_ERR_UNSUPPORTED, fn, "E=%lld exceeds the supported maximum %d", E, kMaxExperts);
  if (k < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "k=%lld must be >= 1", k);
  if (k > E) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "k=%lld exceeds E=%lld", k, E);
  if (k > kMaxTopK) return fail(STRATA_ERR_UNSUPPORTED, fn, "k=%lld exceeds the supported maximum %d", k, kMaxTopK);
  if (T * k >= (1ll << 31)) return fail(STRATA_ERR_UNSUPPORTED, fn, "T*k=%lld must be < 2^31", T * k);
  return STRATA_OK;
}

int check_shape(const char *fn, long long H, long long I, long long g) {
  if (g != 32 && g != 64 && g != 128)
    return fail(STRATA_ERR_UNSUPPORTED, fn, "group=%lld is not one of 32, 64, 128", g);
  if (H < 256 || H > 16384 || H % 256)
    return fail(STRATA_ERR_UNSUPPORTED, fn, "hidden=%lld must be a multiple of 256 in [256, 16384]", H);
  if (I < 128 || I > 16384 || I % 128)
    return fail(STRATA_ERR_UNSUPPORTED, fn, "inter=%lld must be a multiple of 128 in [128, 16384]", I);
  return STRATA_OK;
}

// The weight arrays of `w` for its format: the codes and scales always, the
// zero points (asymmetric 4-bit) or fifth-bit words (5-bit) as the format
// needs them, NULL side arrays otherwise.
int check_weights(const char *fn, const strata_moe_weights *w) {
  REQUIRE_PTR(fn, w->gate);
  REQUIRE_PTR(fn, w->gate_scale);
  REQUIRE_PTR(fn, w->up);
  REQUIRE_PTR(fn, w->up_scale);
  REQUIRE_PTR(fn, w->down);
  REQUIRE_PTR(fn, w->down_scale);
  if (w->layout != STRATA_L_ROWS && w->layout != STRATA_L_TILED)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "layout=%d is not a strata_weight_layout", (int)w->layout);
  const bool zeros = w->gate_zero || w->up_zero || w->down_zero;
  const bool his = w->gate_hi || w->up_hi || w->down_hi;
  switch (w->format) {
    case STRATA_W_INT4:
      if (zeros || his)
        return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "format=STRATA_W_INT4 takes no zero points or fifth-bit words");
      return STRATA_OK;
    case STRATA_W_INT4_ASYM:
      if (his) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "format=STRATA_W_INT4_ASYM takes no fifth-bit words");
      if (!w->gate_zero || !w->up_zero || !w->down_zero)
        return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "format=STRATA_W_INT4_ASYM needs gate_zero, up_zero and down_zero");
      if ((w->hidden / w->group) % 2 || (w->inter / w->group) % 2)
        return fail(STRATA_ERR_UNSUPPORTED, fn,
                    "format=STRATA_W_INT4_ASYM needs an even number of groups per row (hidden=%d, inter=%d, group=%d)",
                    w->hidden, w->inter, w->group);
      return STRATA_OK;
    case STRATA_W_INT5:
      if (zeros) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "format=STRATA_W_INT5 takes no zero points");
      if (!w->gate_hi || !w->up_hi || !w->down_hi)
        return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "format=STRATA_W_INT5 needs gate_hi, up_hi and down_hi");
      for (const void *p : {(const void *)w->gate_hi, (const void *)w->up_hi, (const void *)w->down_hi})
        if (reinterpret_cast<uintptr_t>(p) & 3u)
          return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "fifth-bit words at %p are not 4-byte aligned", p);
      return STRATA_OK;
    default:
      return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "format=%d is not a strata_weight_format", (int)w->format);
  }
}

strata::FfnWeights ffn_weights(const strata_moe_weights *w) {
  strata::FfnWeights fw{w->gate,       w->up,         w->down,   w->gate_scale, w->up_scale,
                        w->down_scale, w->num_experts, w->hidden, w->inter,      w->group};
  fw.fmt = w->format;
  fw.tiled = w->layout == STRATA_L_TILED;
  if (w->format == STRATA_W_INT4_ASYM) {
    fw.gate_x = w->gate_zero;
    fw.up_x = w->up_zero;
    fw.down_x = w->down_zero;
  } else if (w->format == STRATA_W_INT5) {
    fw.gate_x = reinterpret_cast<const uint8_t *>(w->gate_hi);
    fw.up_x = reinterpret_cast<const uint8_t *>(w->up_hi);
    fw.down_x = reinterpret_cast<const uint8_t *>(w->down_hi);
  }
  return fw;
}

enum class FfnPath { Auto, Gemm, Gemv };

// Read on every call (a getenv is negligible next to a kernel launch), so a
// process can switch paths between calls.
FfnPath ffn_path_env() {
  const char *v = std::getenv("STRATA_MOE_FFN_PATH");
  if (!v || !*v || !std::strcmp(v, "auto")) return FfnPath::Auto;
  if (!std::strcmp(v, "gemm")) return FfnPath::Gemm;
  if (!std::strcmp(v, "gemv")) return FfnPath::Gemv;
  return FfnPath::Auto;
}

bool ffn_path_env_valid() {
  const char *v = std::getenv("STRATA_MOE_FFN_PATH");
  return !v || !*v || !std::strcmp(v, "auto") || !std::strcmp(v, "gemm") || !std::strcmp(v, "gemv");
}

}  // namespace

namespace strata {

namespace {
size_t up256(size_t b) { return (b + 255) / 256 * 256; }
// Tiles of the GEMM path: each expert's rows in kGemmRows pieces.
long long max_tiles(long long pairs, int E) {
  return (pairs + kGemmRows - 1) / kGemmRows + std::min<long long>(E, pairs) + 1;
}
}  // namespace

// Regions: xq, h, y16, tiles (two lists), meta (256 B).
size_t ffn_workspace_bytes(long long T, int k, int E, int H, int I) {
  const long long pairs = T * k;
  return up256((size_t)T * H * 2) + up256((size_t)pairs * I * 2) + up256((size_t)pairs * H * 2) +
         up256((size_t)2 * max_tiles(pairs, E) * sizeof(Tile)) + 256;
}

FfnWorkspace carve_ffn_workspace(void *base, long long T, int k, int E, int H, int I) {
  const long long pairs = T * k;
  char *p = static_cast<char *>(base);
  FfnWorkspace w{};
  w.xq = reinterpret_cast<uint16_t *>(p);
  p += up256((size_t)T * H * 2);
  w.h = reinterpret_cast<uint16_t *>(p);
  p += up256((size_t)pairs * I * 2);
  w.y16 = reinterpret_cast<uint16_t *>(p);
  p += up256((size_t)pairs * H * 2);
  w.tiles = reinterpret_cast<Tile *>(p);
  w.tile_cap = max_tiles(pairs, E);
  p += up256((size_t)2 * w.tile_cap * sizeof(Tile));
  w.meta = reinterpret_cast<int *>(p);
  w.bytes = ffn_workspace_bytes(T, k, E, H, I);
  return w;
}

// What strata_moe_workspace_size reports: the ffn regions, then the grouping
// histogram in a region of its own (the layer call's routing kernel writes
// the ffn's fp16 x before the grouping runs).
size_t layer_workspace_bytes(long long T, int E, int k, int H, int I) {
  return up256(ffn_workspace_bytes(T, k, E, H, I)) + up256(permute_workspace_bytes(T * k, E));
}

// ---------------------------------------------------------------- static scratch
// Scratch memory of strata_moe_layer_noalloc, for callers that cannot
// allocate device memory.  Each device the library runs on holds its own copy
// of this array (in the code object's device globals) until the process ends.
// Host code never uses the name `scratch` as an address: it is a host-side
// stand-in; the device address of each device's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = STRATA_MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the scratch array on the device of `stream` (the current
// device for the null stream).  The first call on a device looks it up with
// that device current and restores the caller's current device afterwards.
hipError_t noalloc_scratch(hipStream_t stream, void **out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
    dev = sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace strata

extern "C" {

const char *strata_moe_last_error(void) { return g_last_error.c_str(); }

size_t strata_moe_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I, int32_t g) {
  if (check_tek("strata_moe_workspace_size", T, E, k) != STRATA_OK) return 0;
  if (check_shape("strata_moe_workspace_size", H, I, g) != STRATA_OK) return 0;
  return layer_workspace_bytes(T, E, k, H, I);
}

size_t strata_moe_permute_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (check_tek("strata_moe_permute_workspace_size", T, E, k) != STRATA_OK) return (size_t)-1;
  return permute_workspace_bytes((long long)T * k, E);
}

int strata_moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                     float *topk_w, void *stream) {
  static const char *fn = "strata_moe_route";
  if (int rc = check_tek(fn, T, E, k)) return rc;
  if (T == 0) return ok();
  REQUIRE_PTR(fn, logits);
  REQUIRE_PTR(fn, topk_ids);
  REQUIRE_PTR(fn, topk_w);
  const hipError_t e = launch_route(logits, T, E, k, topk_ids, topk_w, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_moe_router(const uint16_t *x_bf16, int32_t T, int32_t H, const uint16_t *w_router_bf16, int32_t E,
                      int32_t k, float *logits, int32_t *topk_ids, float *topk_w, void *stream) {
  static const char *fn = "strata_moe_router";
  if (int rc = check_tek(fn, T, E, k)) return rc;
  if (H < 64 || H > 16384 || H % 64)
    return fail(STRATA_ERR_UNSUPPORTED, fn, "H=%d must be a multiple of 64 in [64, 16384]", H);
  if ((long long)T * H * 2 >= (1ll << 31) || (long long)E * H * 2 >= (1ll << 31))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "T*H and E*H must stay below 2^30 elements (T=%d, E=%d, H=%d)", T, E, H);
  if (T == 0) return ok();
  REQUIRE_PTR(fn, x_bf16);
  REQUIRE_PTR(fn, w_router_bf16);
  REQUIRE_PTR(fn, logits);
  REQUIRE_PTR(fn, topk_ids);
  REQUIRE_PTR(fn, topk_w);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_router_logits(x_bf16, T, H, w_router_bf16, E, logits, s);
  if (e == hipSuccess) e = launch_route(logits, T, E, k, topk_ids, topk_w, s);
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_moe_permute(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv_perm, void *workspace,
                       size_t workspace_bytes, void *stream) {
  static const char *fn = "strata_moe_permute";
  if (int rc = check_tek(fn, T, E, k)) return rc;
  REQUIRE_PTR(fn, counts);
  REQUIRE_PTR(fn, offsets);
  if (T > 0) {
    REQUIRE_PTR(fn, topk_ids);
    REQUIRE_PTR(fn, perm);
    REQUIRE_PTR(fn, inv_perm);
  }
  const long long pairs = (long long)T * k;
  const size_t need = permute_workspace_bytes(pairs, E);
  if (need > 0) {
    if (workspace == nullptr)
      return fail(STRATA_ERR_WORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "workspace=%p is not 256-byte aligned", workspace);
    if (workspace_bytes < need)
      return fail(STRATA_ERR_WORKSPACE, fn, "workspace_bytes=%zu is smaller than the required %zu", workspace_bytes, need);
  }
  // T == 0 still defines counts = 0 and offsets = 0 (the small path handles it).
  const hipError_t e = launch_permute(topk_ids, (int)pairs, E, counts, offsets, perm, inv_perm, workspace,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_moe_ffn(const uint16_t *x_bf16, int32_t T, int32_t k, const strata_moe_weights *w,
                   const int32_t *offsets, const int32_t *perm, const float *topk_w, float *y_or_out,
                   void *workspace, size_t workspace_bytes, void *stream) {
  static const char *fn = "strata_moe_ffn";
  if (w == nullptr) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "w is NULL");
  if (int rc = check_tek(fn, T, w->num_experts, k)) return rc;
  if (int rc = check_shape(fn, w->hidden, w->inter, w->group)) return rc;
  if (!ffn_path_env_valid())
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "STRATA_MOE_FFN_PATH=%s is not one of auto, gemm, gemv",
                std::getenv("STRATA_MOE_FFN_PATH"));
  if (T == 0) return ok();
  REQUIRE_PTR(fn, x_bf16);
  REQUIRE_PTR(fn, offsets);
  REQUIRE_PTR(fn, perm);
  REQUIRE_PTR(fn, y_or_out);
  if (int rc = check_weights(fn, w)) return rc;
  if (topk_w != nullptr && !aligned16(topk_w))
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "topk_w=%p is not 16-byte aligned", (const void *)topk_w);
  const int E = w->num_experts, H = w->hidden, I = w->inter, g = w->group;
  const size_t need = ffn_workspace_bytes(T, k, E, H, I);
  if (workspace == nullptr)
    return fail(STRATA_ERR_WORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "workspace=%p is not 256-byte aligned", workspace);
  if (workspace_bytes < need)
    return fail(STRATA_ERR_WORKSPACE, fn, "workspace_bytes=%zu is smaller than the required %zu", workspace_bytes, need);

  const FfnPath forced = ffn_path_env();
  const bool gemv_ok = gemv_supported(T, H, I);
  if (forced == FfnPath::Gemv && !gemv_ok)
    return fail(STRATA_ERR_UNSUPPORTED, fn,
                "STRATA_MOE_FFN_PATH=gemv needs T <= %d, hidden in {256,512,1024,2048,4096} and inter a power of two "
                "in [128, 2048] (T=%d, hidden=%d, inter=%d)",
                kGemvMaxTokens, T, H, I);
  const bool use_gemv = forced == FfnPath::Gemv || (forced == FfnPath::Auto && gemv_ok);

  const FfnWeights fw = ffn_weights(w);
  const FfnWorkspace ws = carve_ffn_workspace(workspace, T, k, E, H, I);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = use_gemv ? launch_ffn_gemv(x_bf16, T, k, fw, offsets, perm, topk_w, y_or_out, ws, s)
                                : launch_ffn_gemm(x_bf16, T, k, fw, offsets, perm, topk_w, y_or_out, ws, s);
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

// The layer call on a given workspace (strata_moe_layer and
// strata_moe_layer_noalloc); `fn` names the entry point in error messages.
static int layer_impl(const char *fn, const float *logits, const uint16_t *x_bf16, int32_t T, int32_t k,
                      const strata_moe_weights *w, int32_t *topk_ids, float *topk_w, int32_t *counts,
                      int32_t *offsets, int32_t *perm, int32_t *inv_perm, float *out, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (w == nullptr) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "w is NULL");
  const int E = w->num_experts, H = w->hidden, I = w->inter, g = w->group;
  if (int rc = check_tek(fn, T, E, k)) return rc;
  if (int rc = check_shape(fn, H, I, g)) return rc;
  if (!ffn_path_env_valid())
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "STRATA_MOE_FFN_PATH=%s is not one of auto, gemm, gemv",
                std::getenv("STRATA_MOE_FFN_PATH"));
  REQUIRE_PTR(fn, counts);
  REQUIRE_PTR(fn, offsets);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {  // counts = 0 and offsets = 0, as strata_moe_permute defines them
    const hipError_t e = launch_permute(nullptr, 0, E, counts, offsets, nullptr, nullptr, nullptr, s);
    return e == hipSuccess ? ok() : hip_fail(fn, e);
  }
  REQUIRE_PTR(fn, logits);
  REQUIRE_PTR(fn, x_bf16);
  REQUIRE_PTR(fn, topk_ids);
  REQUIRE_PTR(fn, topk_w);
  REQUIRE_PTR(fn, perm);
  REQUIRE_PTR(fn, inv_perm);
  REQUIRE_PTR(fn, out);
  if (int rc = check_weights(fn, w)) return rc;
  const long long pairs = (long long)T * k;
  const size_t need = layer_workspace_bytes(T, E, k, H, I);
  if (workspace == nullptr)
    return fail(STRATA_ERR_WORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "workspace=%p is not 256-byte aligned", workspace);
  if (workspace_bytes < need)
    return fail(STRATA_ERR_WORKSPACE, fn, "workspace_bytes=%zu is smaller than the required %zu", workspace_bytes, need);

  const FfnPath forced = ffn_path_env();
  const bool gemv_ok = gemv_supported(T, H, I);
  if (forced == FfnPath::Gemv && !gemv_ok)
    return fail(STRATA_ERR_UNSUPPORTED, fn,
                "STRATA_MOE_FFN_PATH=gemv needs T <= %d, hidden in {256,512,1024,2048,4096} and inter a power of two "
                "in [128, 2048] (T=%d, hidden=%d, inter=%d)",
                kGemvMaxTokens, T, H, I);
  const FfnWeights fw = ffn_weights(w);
  const FfnWorkspace ws = carve_ffn_workspace(workspace, T, k, E, H, I);
  hipError_t e;
  if (forced != FfnPath::Gemm && decode_layer_supported(T, E, k, H, I)) {
    e = launch_decode_layer(logits, x_bf16, T, k, fw, topk_ids, topk_w, counts, offsets, perm, inv_perm, out, ws, s);
  } else {
    const bool use_gemv = forced == FfnPath::Gemv || (forced == FfnPath::Auto && gemv_ok);
    if (!use_gemv && pairs > kPermuteSmallMax) {
      // Grouped-GEMM path in six kernels: the routing kernel also converts x,
      // the grouping scan also builds the tile lists (no prologue kernel).
      void *hist = static_cast<char *>(workspace) + (ffn_workspace_bytes(T, k, E, H, I) + 255) / 256 * 256;
      e = launch_route_convert(logits, T, E, k, topk_ids, topk_w, x_bf16, ws.xq, (size_t)T * H / 8, s);
      if (e == hipSuccess)
        e = launch_permute(topk_ids, (int)pairs, E, counts, offsets, perm, inv_perm, hist, s, ws.tiles,
                           ws.tiles + ws.tile_cap, ws.meta);
      if (e == hipSuccess) e = launch_ffn_gemm(x_bf16, T, k, fw, offsets, perm, topk_w, out, ws, s, true);
    } else {
      e = launch_route(logits, T, E, k, topk_ids, topk_w, s);
      if (e == hipSuccess) e = launch_permute(topk_ids, (int)pairs, E, counts, offsets, perm, inv_perm, workspace, s);
      if (e == hipSuccess)
        e = use_gemv ? launch_ffn_gemv(x_bf16, T, k, fw, offsets, perm, topk_w, out, ws, s)
                     : launch_ffn_gemm(x_bf16, T, k, fw, offsets, perm, topk_w, out, ws, s);
    }
  }
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_moe_layer(const float *logits, const uint16_t *x_bf16, int32_t T, int32_t k, const strata_moe_weights *w,
                     int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets, int32_t *perm,
                     int32_t *inv_perm, float *out, void *workspace, size_t workspace_bytes, void *stream) {
  return layer_impl("strata_moe_layer", logits, x_bf16, T, k, w, topk_ids, topk_w, counts, offsets, perm, inv_perm,
                    out, workspace, workspace_bytes, stream);
}

int strata_moe_layer_noalloc(const float *logits, const uint16_t *x_bf16, int32_t T, int32_t k,
                             const strata_moe_weights *w, int32_t *topk_ids, float *topk_w, int32_t *counts,
                             int32_t *offsets, int32_t *perm, int32_t *inv_perm, float *out, void *stream) {
  static const char *fn = "strata_moe_layer_noalloc";
  if (w == nullptr) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "w is NULL");
  if (int rc = check_tek(fn, T, w->num_experts, k)) return rc;
  if (int rc = check_shape(fn, w->hidden, w->inter, w->group)) return rc;
  const size_t need = layer_workspace_bytes(T, w->num_experts, k, w->hidden, w->inter);
  if (need > kNoAllocScratchBytes)
    return fail(STRATA_ERR_UNSUPPORTED, fn,
                "T=%d, E=%d, k=%d, hidden=%d, inter=%d needs %zu bytes of scratch, more than the library's static "
                "%zu (STRATA_MOE_NOALLOC_SCRATCH_BYTES); call strata_moe_layer with a workspace instead",
                T, w->num_experts, k, w->hidden, w->inter, need, kNoAllocScratchBytes);
  void *ws = nullptr;
  const hipError_t e = noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) return hip_fail(fn, e);
  return layer_impl(fn, logits, x_bf16, T, k, w, topk_ids, topk_w, counts, offsets, perm, inv_perm, out, ws,
                    kNoAllocScratchBytes, stream);
}

int strata_moe_combine(const float *y, const int32_t *inv_perm, const float *topk_w, int32_t T, int32_t k,
                       int32_t H, float *out, void *stream) {
  static const char *fn = "strata_moe_combine";
  if (T < 0) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "T=%d is negative", T);
  if (k < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "k=%d must be >= 1", k);
  if (k > kMaxTopK) return fail(STRATA_ERR_UNSUPPORTED, fn, "k=%d exceeds the supported maximum %d", k, kMaxTopK);
  if (H < 4 || H % 4) return fail(STRATA_ERR_UNSUPPORTED, fn, "H=%d must be a positive multiple of 4", H);
  if ((long long)T * k >= (1ll << 31)) return fail(STRATA_ERR_UNSUPPORTED, fn, "T*k=%lld must be < 2^31", (long long)T * k);
  if (T == 0) return ok();
  REQUIRE_PTR(fn, y);
  REQUIRE_PTR(fn, inv_perm);
  REQUIRE_PTR(fn, topk_w);
  REQUIRE_PTR(fn, out);
  const hipError_t e = launch_combine(y, inv_perm, topk_w, T, k, H, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_kv_quantize(const uint16_t *x_bf16, int32_t T, int32_t Hkv, int32_t D, const int32_t *slots,
                       uint8_t *codes, uint16_t *scales, int32_t L, void *stream) {
  static const char *fn = "strata_kv_quantize";
  if (T < 0) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "T=%d is negative", T);
  if (L < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "L=%d must be >= 1", L);
  if (!kv_shape_supported(Hkv, D))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "Hkv=%d, D=%d: supported are D = 128 and Hkv in {1, 2, 4, 8}", Hkv, D);
  if ((long long)T * Hkv >= (1ll << 31) || (long long)L * Hkv * D >= (1ll << 40))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "T=%d or L=%d too large", T, L);
  if (T == 0) return ok();
  REQUIRE_PTR(fn, x_bf16);
  REQUIRE_PTR(fn, slots);
  REQUIRE_PTR(fn, codes);
  REQUIRE_PTR(fn, scales);
  const hipError_t e = launch_kv_quantize(x_bf16, T, Hkv, slots, L, codes, scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_kv_quantize_pair(const uint16_t *k_bf16, const uint16_t *v_bf16, int32_t T, int32_t Hkv, int32_t D,
                            const int32_t *slots, uint8_t *k_codes, uint16_t *k_scales, uint8_t *v_codes,
                            uint16_t *v_scales, int32_t L, void *stream) {
  static const char *fn = "strata_kv_quantize_pair";
  if (T < 0) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "T=%d is negative", T);
  if (L < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "L=%d must be >= 1", L);
  if (!kv_shape_supported(Hkv, D))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "Hkv=%d, D=%d: supported are D = 128 and Hkv in {1, 2, 4, 8}", Hkv, D);
  if ((long long)T * Hkv * 2 >= (1ll << 31) || (long long)L * Hkv * D >= (1ll << 40))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "T=%d or L=%d too large", T, L);
  if (T == 0) return ok();
  REQUIRE_PTR(fn, k_bf16);
  REQUIRE_PTR(fn, v_bf16);
  REQUIRE_PTR(fn, slots);
  REQUIRE_PTR(fn, k_codes);
  REQUIRE_PTR(fn, k_scales);
  REQUIRE_PTR(fn, v_codes);
  REQUIRE_PTR(fn, v_scales);
  const hipError_t e = launch_kv_quantize(k_bf16, T, Hkv, slots, L, k_codes, k_scales,
                                          static_cast<hipStream_t>(stream), v_bf16, v_codes, v_scales);
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_moe_tile_weights(const uint8_t *src, uint8_t *dst, int64_t rows, int32_t K, void *stream) {
  static const char *fn = "strata_moe_tile_weights";
  if (rows < 0 || rows % 32)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "rows=%lld must be a non-negative multiple of 32", (long long)rows);
  if (K < 128 || K % 128) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "K=%d must be a positive multiple of 128", K);
  if (rows == 0) return ok();
  REQUIRE_PTR(fn, src);
  REQUIRE_PTR(fn, dst);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t n = (uintptr_t)rows * (uintptr_t)(K / 2);
  if (a < b + n && b < a + n) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "src=%p and dst=%p overlap", src, dst);
  const hipError_t e = launch_tile_weights(src, dst, rows, K, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

size_t strata_sparse_attention_workspace_size(int32_t Tq, int32_t Hq, int32_t n_sel) {
  if (Tq < 0 || Hq < 1 || n_sel < 1) return 0;
  return attn_workspace_bytes(Tq, Hq, n_sel);
}

int strata_sparse_attention(const uint16_t *q_bf16, int32_t Tq, int32_t Hq, const uint8_t *k_codes,
                            const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales, int32_t L,
                            int32_t Hkv, int32_t D, const int32_t *sel, int32_t n_sel, float sm_scale, float *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
  static const char *fn = "strata_sparse_attention";
  if (Tq < 0) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "Tq=%d is negative", Tq);
  if (L < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "L=%d must be >= 1", L);
  if (n_sel < 1) return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "n_sel=%d must be >= 1", n_sel);
  if (n_sel > 32768) return fail(STRATA_ERR_UNSUPPORTED, fn, "n_sel=%d exceeds the supported maximum 32768", n_sel);
  if (sel == nullptr && n_sel > L)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "sel is NULL and n_sel=%d exceeds L=%d", n_sel, L);
  if (!kv_shape_supported(Hkv, D))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "Hkv=%d, D=%d: supported are D = 128 and Hkv in {1, 2, 4, 8}", Hkv, D);
  if (Hq < Hkv || Hq % Hkv || Hq / Hkv > 4)
    return fail(STRATA_ERR_UNSUPPORTED, fn, "Hq=%d must be Hkv=%d times 1, 2 or 4", Hq, Hkv);
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "sm_scale is not finite");
  if ((long long)Tq * ((n_sel + 31) / 32) >= (1ll << 31) || (long long)L * Hkv * D >= (1ll << 40))
    return fail(STRATA_ERR_UNSUPPORTED, fn, "Tq=%d, n_sel=%d or L=%d too large", Tq, n_sel, L);
  if (Tq == 0) return ok();
  REQUIRE_PTR(fn, q_bf16);
  REQUIRE_PTR(fn, k_codes);
  REQUIRE_PTR(fn, k_scales);
  REQUIRE_PTR(fn, v_codes);
  REQUIRE_PTR(fn, v_scales);
  REQUIRE_PTR(fn, out);
  if (sel != nullptr && !aligned16(sel))
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "sel=%p is not 16-byte aligned", (const void *)sel);
  const size_t need = attn_workspace_bytes(Tq, Hq, n_sel);
  if (workspace == nullptr)
    return fail(STRATA_ERR_WORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "workspace=%p is not 256-byte aligned", workspace);
  if (workspace_bytes < need)
    return fail(STRATA_ERR_WORKSPACE, fn, "workspace_bytes=%zu is smaller than the required %zu", workspace_bytes, need);
  const hipError_t e = launch_sparse_attention(q_bf16, Tq, Hq, k_codes, k_scales, v_codes, v_scales, L, Hkv, sel,
                                               n_sel, sm_scale, out, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

int strata_moe_timing_enable(int32_t on) {
  timing_enable(on);
  return ok();
}

int strata_moe_timing_query(const char *kernel, int32_t *launches, double *total_ms) {
  static const char *fn = "strata_moe_timing_query";
  if (launches == nullptr || total_ms == nullptr)
    return fail(STRATA_ERR_INVALID_ARGUMENT, fn, "launches and total_ms must not be NULL");
  int n = 0;
  double ms = 0.0;
  if (timing_query(kernel, &n, &ms) != 0) return fail(STRATA_ERR_HIP, fn, "waiting for timing events failed");
  *launches = n;
  *total_ms = ms;
  return ok();
}

int32_t strata_moe_timing_kernels(const char **names, int32_t max_names) {
  return timing_names(names, names ? max_names : 0);
}

}  // extern "C"
