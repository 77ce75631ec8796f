// C ABI of the sparse gated-FFN library: argument validation, workspace sizing and
// dispatch to the HIP kernels. Every argument is checked before any HIP call, so the
// error paths run (and are tested) on machines without a GPU.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <exception>

#include "kernels.h"
#include "sparse_ffn.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
// 4-byte alignment of an optional int32 or fp32 pointer (NULL passes)
bool aligned4_or_null(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int wbytes(int wdtype) { return wdtype == SFN_BF16 ? 2 : 4; }

// Shape, enum and alignment checks shared by every call on an FFN layer.
int check_ffn(const sfn_ffn* ffn, bool need_up_down) {
  if (!ffn) return SFN_EINVAL;
  if (ffn->wdtype != SFN_F32 && ffn->wdtype != SFN_BF16) return SFN_EDTYPE;
  if (ffn->act != SFN_ACT_SILU && ffn->act != SFN_ACT_RELU) return SFN_EINVAL;
  if (ffn->d < 1 || ffn->d > SFN_MAX_D || ffn->f < 1 || ffn->f > SFN_MAX_F) return SFN_ESHAPE;
  if ((ffn->d * wbytes(ffn->wdtype)) % 16 != 0) return SFN_EALIGN;
  if (!ffn->w_gate) return SFN_EINVAL;
  if (need_up_down && (!ffn->w_up || !ffn->w_down_t)) return SFN_EINVAL;
  if (!aligned16(ffn->w_gate)) return SFN_EALIGN;
  if (ffn->w_up && !aligned16(ffn->w_up)) return SFN_EALIGN;
  if (ffn->w_down_t && !aligned16(ffn->w_down_t)) return SFN_EALIGN;
  if (ffn->b_gate && (reinterpret_cast<uintptr_t>(ffn->b_gate) & 3u)) return SFN_EALIGN;
  return SFN_OK;
}

int check_svd(const sfn_svd* s) {
  if (!s) return SFN_EINVAL;
  if (s->reserved != 0) return SFN_EINVAL;
  if (s->d < 1 || s->d > SFN_MAX_D || s->f < 1 || s->f > SFN_MAX_F) return SFN_ESHAPE;
  if (s->r < 1 || s->r > SFN_MAX_RANK || s->r > s->d) return SFN_ESHAPE;
  if (s->d % 8 != 0 || s->r % 8 != 0) return SFN_EALIGN;
  if (!s->q || !s->l || !s->tau) return SFN_EINVAL;
  if (!aligned16(s->q) || !aligned16(s->l)) return SFN_EALIGN;
  if ((reinterpret_cast<uintptr_t>(s->tau) & 3u) || (s->b && (reinterpret_cast<uintptr_t>(s->b) & 3u)))
    return SFN_EALIGN;
  return SFN_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return SFN_EWORKSPACE;
  if (!aligned256(ws)) return SFN_EALIGN;
  return SFN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SFN_OK : SFN_EHIP; }

// Validation and launch of one decode step on a workspace (sparse_ffn_decode and its
// allocation-free variant).
int decode_validate(const sfn_ffn* ffn, const void* x, int32_t B, const float* t, const int32_t* cand,
                    const int32_t* n_cand, const uint8_t* mask_in, float* y, const int32_t* active_idx,
                    const int32_t* n_active) {
  const int st = check_ffn(ffn, y != nullptr);
  if (st != SFN_OK) return st;
  if (!x) return SFN_EINVAL;
  if (!aligned16(x)) return SFN_EALIGN;
  if (B < 1 || B > SFN_MAX_BATCH) return SFN_ESHAPE;
  if ((cand == nullptr) != (n_cand == nullptr)) return SFN_EINVAL;
  if (cand && (B != 1 || mask_in)) return SFN_EINVAL;
  if (y && !aligned16(y)) return SFN_EALIGN;
  if (!aligned4_or_null(t) || !aligned4_or_null(cand) || !aligned4_or_null(n_cand) ||
      !aligned4_or_null(active_idx) || !aligned4_or_null(n_active))
    return SFN_EALIGN;
  return SFN_OK;
}

size_t decode_need(const sfn_ffn* ffn, int32_t B) {
  return sfn::decode_workspace_bytes(ffn->d, ffn->f, wbytes(ffn->wdtype), B > 1 ? SFN_MAX_BATCH : 1);
}

int decode_launch(const sfn_ffn* ffn, const void* x, int32_t B, const float* t, const int32_t* cand,
                  const int32_t* n_cand, const uint8_t* mask_in, float* y, int32_t* active_idx, int32_t* n_active,
                  void* ws, void* stream) {
  const int wb = wbytes(ffn->wdtype);
  sfn::DecodeArgs a{};
  a.wg = static_cast<const char*>(ffn->w_gate);
  a.wu = static_cast<const char*>(ffn->w_up);
  a.wd = static_cast<const char*>(ffn->w_down_t);
  a.bias = ffn->b_gate;
  a.x = static_cast<const char*>(x);
  a.t = t;
  a.cand = cand;
  a.n_cand = n_cand;
  a.mask_in = mask_in;
  a.y = y;
  a.active_idx = active_idx;
  a.n_active = n_active;
  a.d = ffn->d;
  a.f = ffn->f;
  a.nch = ffn->d * wb / 16;
  a.row_bytes = ffn->d * wb;
  a.nb = B;
  a.act = ffn->act;
  a.G = sfn::decode_grid(ffn->f);
  a.n_red = sfn::decode_reducers(a.G, B, ffn->d);
  sfn::decode_carve(a, ws, wb);
  return hip_status(sfn::launch_decode(a, ffn->wdtype, static_cast<hipStream_t>(stream)));
}

// Scratch of sparse_ffn_decode_noalloc: a file-scope device array, one copy on each GPU
// the library runs on, zero when the code object is loaded. Kernels never see its name:
// host code takes its device address from hipGetSymbolAddress, once per device with that
// device current, and passes that address like a workspace.
constexpr size_t kNoAllocScratchBytes = SFN_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (resolved on the first call on each device;
// host threads that race store the same value).
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SFN_EHIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SFN_EHIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SFN_OK;
}

}  // namespace

extern "C" {

size_t sparse_ffn_workspace_size(const sfn_ffn* ffn, int32_t max_tokens) {
  try {
    if (check_ffn(ffn, false) != SFN_OK || max_tokens < 1 || max_tokens > 65536) return 0;
    const int wb = wbytes(ffn->wdtype);
    const int nb = max_tokens > 1 ? SFN_MAX_BATCH : 1;
    size_t need = sfn::decode_workspace_bytes(ffn->d, ffn->f, wb, nb);
    const size_t chunk = sfn::chunk_workspace_bytes(ffn->d, ffn->f, ffn->wdtype, max_tokens < SFN_MAX_CHUNK ? max_tokens : SFN_MAX_CHUNK);
    if (chunk > need) need = chunk;
    const size_t cal = sfn::calibrate_workspace_bytes(ffn->d, ffn->f, ffn->wdtype, max_tokens);
    if (cal > need) need = cal;
    return need;
  } catch (...) {
    return 0;
  }
}

size_t svd_predict_workspace_size(const sfn_svd* svd) {
  try {
    if (check_svd(svd) != SFN_OK) return 0;
    return sfn::svd_workspace_bytes(svd->d, svd->f, svd->r);
  } catch (...) {
    return 0;
  }
}

const char* sparse_ffn_strerror(int status) {
  switch (status) {
    case SFN_OK: return "success";
    case SFN_EINVAL: return "invalid argument (null pointer, bad enum or out-of-range scalar)";
    case SFN_ESHAPE: return "unsupported shape (d, f, r, batch or chunk size out of range)";
    case SFN_EDTYPE: return "unsupported dtype";
    case SFN_EWORKSPACE: return "workspace missing or smaller than the size query returns";
    case SFN_EALIGN: return "pointer or row not 16-byte aligned (workspace: 256-byte)";
    case SFN_EUNSUPPORTED: return "request not implemented by this library";
    case SFN_EHIP: return "HIP runtime error on launch";
    case SFN_ETOOLARGE:
      return "request needs more scratch than sparse_ffn_decode_noalloc's fixed array (SFN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int sparse_ffn_decode(const sfn_ffn* ffn, const void* x, int32_t B, const float* t, const int32_t* cand,
                      const int32_t* n_cand, const uint8_t* mask_in, float* y, int32_t* active_idx,
                      int32_t* n_active, void* ws, size_t ws_bytes, void* stream) {
  try {
    int st = decode_validate(ffn, x, B, t, cand, n_cand, mask_in, y, active_idx, n_active);
    if (st != SFN_OK) return st;
    st = check_ws(ws, ws_bytes, decode_need(ffn, B));
    if (st != SFN_OK) return st;
    return decode_launch(ffn, x, B, t, cand, n_cand, mask_in, y, active_idx, n_active, ws, stream);
  } catch (...) {
    return SFN_EHIP;
  }
}

int sparse_ffn_decode_noalloc(const sfn_ffn* ffn, const void* x, int32_t B, const float* t, const int32_t* cand,
                              const int32_t* n_cand, const uint8_t* mask_in, float* y, int32_t* active_idx,
                              int32_t* n_active, void* stream) {
  try {
    int st = decode_validate(ffn, x, B, t, cand, n_cand, mask_in, y, active_idx, n_active);
    if (st != SFN_OK) return st;
    if (decode_need(ffn, B) > kNoAllocScratchBytes) return SFN_ETOOLARGE;
    void* ws = nullptr;
    st = scratch_ptr(&ws);
    if (st != SFN_OK) return st;
    return decode_launch(ffn, x, B, t, cand, n_cand, mask_in, y, active_idx, n_active, ws, stream);
  } catch (...) {
    return SFN_EHIP;
  }
}

int sparse_ffn_decode_parallel(const sfn_ffn* ffn, const void* x, const int32_t* cand, const int32_t* n_cand,
                               float* y, void* ws, size_t ws_bytes, void* stream) {
  try {
    int st = check_ffn(ffn, true);
    if (st != SFN_OK) return st;
    if (!x || !cand || !n_cand || !y) return SFN_EINVAL;
    if (!aligned16(x) || !aligned16(y)) return SFN_EALIGN;
    if (!aligned4_or_null(cand) || !aligned4_or_null(n_cand)) return SFN_EALIGN;
    const int wb = wbytes(ffn->wdtype);
    st = check_ws(ws, ws_bytes, sfn::decode_workspace_bytes(ffn->d, ffn->f, wb, 1));
    if (st != SFN_OK) return st;

    sfn::DecodeArgs a{};
    a.wg = static_cast<const char*>(ffn->w_gate);
    a.wu = static_cast<const char*>(ffn->w_up);
    a.wd = static_cast<const char*>(ffn->w_down_t);
    a.bias = ffn->b_gate;
    a.x = static_cast<const char*>(x);
    a.cand = cand;
    a.n_cand = n_cand;
    a.y = y;
    a.d = ffn->d;
    a.f = ffn->f;
    a.nch = ffn->d * wb / 16;
    a.row_bytes = ffn->d * wb;
    a.nb = 1;
    a.act = ffn->act;
    a.G = sfn::decode_grid(ffn->f);
    a.n_red = sfn::decode_reducers(a.G, 1, ffn->d);
    sfn::decode_carve(a, ws, wb);
    return hip_status(sfn::launch_decode_parallel(a, ffn->wdtype, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return SFN_EHIP;
  }
}

int sparse_ffn_calibrate(const sfn_ffn* ffn, const void* x_cal, int32_t n, float k, float* t_out,
                         float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  try {
    int st = check_ffn(ffn, false);
    if (st != SFN_OK) return st;
    if (!x_cal || !t_out) return SFN_EINVAL;
    if (!aligned16(x_cal)) return SFN_EALIGN;
    if (n < 1 || n > 65536) return SFN_ESHAPE;
    if (!(k >= 0.0f && k <= 1.0f)) return SFN_EINVAL;
    if ((int64_t)n * ffn->f > (int64_t)1 << 31) return SFN_ESHAPE;
    if (scores_out && (reinterpret_cast<uintptr_t>(scores_out) & 15u)) return SFN_EALIGN;
    st = check_ws(ws, ws_bytes, sfn::calibrate_workspace_bytes(ffn->d, ffn->f, ffn->wdtype, n));
    if (st != SFN_OK) return st;
    return hip_status(sfn::launch_calibrate(*ffn, x_cal, n, k, t_out, scores_out, ws, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return SFN_EHIP;
  }
}

int svd_predict(const sfn_svd* svd, const void* x, int32_t* cand_idx, int32_t* n_cand, float* p_out, void* ws,
                size_t ws_bytes, void* stream) {
  try {
    int st = check_svd(svd);
    if (st != SFN_OK) return st;
    if (!x || !cand_idx || !n_cand) return SFN_EINVAL;
    if (!aligned16(x)) return SFN_EALIGN;
    if (p_out && (reinterpret_cast<uintptr_t>(p_out) & 3u)) return SFN_EALIGN;
    st = check_ws(ws, ws_bytes, sfn::svd_workspace_bytes(svd->d, svd->f, svd->r));
    if (st != SFN_OK) return st;
    return hip_status(sfn::launch_svd_predict(*svd, x, cand_idx, n_cand, p_out, ws, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return SFN_EHIP;
  }
}

namespace {

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Fused SVD pipeline workspace: the decode scratch for one token, then z [r] fp32.
size_t svd_pipeline_z_offset(const sfn_ffn* ffn) { return round256(sfn::decode_workspace_bytes(ffn->d, ffn->f, 2, 1)); }
size_t svd_pipeline_bytes(const sfn_ffn* ffn, const sfn_svd* svd) {
  return svd_pipeline_z_offset(ffn) + round256((size_t)svd->r * sizeof(float));
}

int check_svd_pipeline(const sfn_ffn* ffn, const sfn_svd* svd) {
  int st = check_ffn(ffn, true);
  if (st != SFN_OK) return st;
  st = check_svd(svd);
  if (st != SFN_OK) return st;
  if (ffn->wdtype != SFN_BF16) return SFN_EDTYPE;  // the predictor takes the bf16 token
  if (svd->d != ffn->d || svd->f != ffn->f) return SFN_ESHAPE;
  return SFN_OK;
}

}  // namespace

size_t sparse_ffn_svd_workspace_size(const sfn_ffn* ffn, const sfn_svd* svd) {
  try {
    if (check_svd_pipeline(ffn, svd) != SFN_OK) return 0;
    return svd_pipeline_bytes(ffn, svd);
  } catch (...) {
    return 0;
  }
}

int sparse_ffn_decode_svd(const sfn_ffn* ffn, const sfn_svd* svd, const void* x, int32_t pipeline, float* y,
                          int32_t* idx, int32_t* n_idx, void* ws, size_t ws_bytes, void* stream) {
  try {
    int st = check_svd_pipeline(ffn, svd);
    if (st != SFN_OK) return st;
    if (!x) return SFN_EINVAL;
    if (pipeline != SFN_PIPE_SEQUENTIAL && pipeline != SFN_PIPE_PARALLEL) return SFN_EINVAL;
    if (pipeline == SFN_PIPE_PARALLEL && !y) return SFN_EINVAL;
    if (!y && !idx && !n_idx) return SFN_EINVAL;  // nothing to compute
    if (!aligned16(x)) return SFN_EALIGN;
    if (y && !aligned16(y)) return SFN_EALIGN;
    if ((idx && (reinterpret_cast<uintptr_t>(idx) & 3u)) || (n_idx && (reinterpret_cast<uintptr_t>(n_idx) & 3u)))
      return SFN_EALIGN;
    st = check_ws(ws, ws_bytes, svd_pipeline_bytes(ffn, svd));
    if (st != SFN_OK) return st;

    float* z = reinterpret_cast<float*>(static_cast<char*>(ws) + svd_pipeline_z_offset(ffn));
    sfn::DecodeArgs a{};
    a.wg = static_cast<const char*>(ffn->w_gate);
    a.wu = static_cast<const char*>(ffn->w_up);
    a.wd = static_cast<const char*>(ffn->w_down_t);
    a.bias = ffn->b_gate;
    a.x = static_cast<const char*>(x);
    a.y = y;
    a.active_idx = idx;
    a.n_active = n_idx;
    a.pl = static_cast<const char*>(svd->l);
    a.pz = z;
    a.ptau = svd->tau;
    a.pb = svd->b;
    a.pr = svd->r;
    a.d = ffn->d;
    a.f = ffn->f;
    a.nch = ffn->d * 2 / 16;
    a.row_bytes = ffn->d * 2;
    a.nb = 1;
    a.act = ffn->act;
    a.G = sfn::decode_grid(ffn->f);
    a.n_red = sfn::decode_reducers(a.G, 1, ffn->d);
    sfn::decode_carve(a, ws, 2);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sfn::launch_svd_z(*svd, x, z, s);
    if (e != hipSuccess) return SFN_EHIP;
    e = pipeline == SFN_PIPE_PARALLEL ? sfn::launch_decode_parallel(a, SFN_BF16, s) : sfn::launch_decode(a, SFN_BF16, s);
    return hip_status(e);
  } catch (...) {
    return SFN_EHIP;
  }
}

int ffn_dense_chunk(const sfn_ffn* ffn, const void* x, int32_t n, float* y, void* ws, size_t ws_bytes,
                    void* stream) {
  try {
    int st = check_ffn(ffn, true);
    if (st != SFN_OK) return st;
    if (!x || !y) return SFN_EINVAL;
    if (!aligned16(x) || !aligned16(y)) return SFN_EALIGN;
    if (n < 1 || n > SFN_MAX_CHUNK) return SFN_ESHAPE;
    st = check_ws(ws, ws_bytes, sfn::chunk_workspace_bytes(ffn->d, ffn->f, ffn->wdtype, n));
    if (st != SFN_OK) return st;
    return hip_status(sfn::launch_dense_chunk(*ffn, x, n, y, ws, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return SFN_EHIP;
  }
}

}  // extern "C"
