// fa_api.hip — the extern "C" entry points declared in include/fa.h: argument checks, then launches.
//
// Every check runs before any HIP call, so a rejected call enqueues nothing and needs no GPU.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Shape limits: per-head tensors are addressed with 32-bit byte offsets by the kernels' buffer loads
// (one extra tile of headroom), grids are 32-bit, and B·H·N·d stays below 2^40.
fa_status check_shape(int B, int H, int N, int d, size_t elem_bytes) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  const uint64_t per_head = (uint64_t)(N + 256) * (uint64_t)d * elem_bytes;
  if (per_head >= (1ull << 31)) return FA_ERR_SHAPE;
  const uint64_t total = (uint64_t)B * (uint64_t)H * (uint64_t)N * (uint64_t)d;
  if (total >= (1ull << 40)) return FA_ERR_SHAPE;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)((N + 63) / 64) >= (1ull << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

bool good_scale(float s) { return isfinite(s) && s > 0.f; }

}  // namespace

extern "C" {

fa_status fa_device_info(int device, int* compute_units, int* peak_clock_khz) {
  if (compute_units == nullptr || peak_clock_khz == nullptr) return FA_ERR_NULL;
  int cus = 0, khz = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device) != hipSuccess)
    return FA_ERR_LAUNCH;
  *compute_units = cus;
  *peak_clock_khz = khz;
  return FA_OK;
}

const char* fa_status_str(fa_status status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H, N (or Nq, Nk) out of range";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension, scale or descale not supported";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not suitably aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
  }
  return "unknown fa_status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, N, d, 2);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 16))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, causal ? 1 : 0, softmax_scale};
  return fa::launch_fwd_bf16(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int causal) {
  if (check_shape(B, H, N, d, 2) != FA_OK) return 0;
  return fa::fwd_split_workspace_bytes(B, H, N, d, causal ? 1 : 0);
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, N, d, 2);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 16))
    return FA_ERR_ALIGN;
  const size_t need = fa::fwd_split_workspace_bytes(B, H, N, d, causal ? 1 : 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, causal ? 1 : 0, softmax_scale};
  a.workspace = need > 0 ? workspace : nullptr;
  return fa::launch_fwd_bf16(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale,
                     float k_descale, float v_descale, void* o, float* lse, int B, int H, int N,
                     int d, int causal, float softmax_scale, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, N, d, 2);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale) || !good_scale(q_descale) || !good_scale(k_descale) ||
      !good_scale(v_descale))
    return FA_ERR_UNSUPPORTED;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) ||
      !aligned(lse, 16))
    return FA_ERR_ALIGN;
  fa::Fp8FwdArgs a{q8, k8, v8, q_descale, k_descale, v_descale, o, lse,
                   B, H, N, d, causal ? 1 : 0, softmax_scale};
  return fa::launch_fwd_fp8(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_fwd_fp8_split(const void* q8, const void* k8, const void* v8, float q_descale,
                           float k_descale, float v_descale, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d, int causal,
                           float softmax_scale, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, N, d, 2);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale) || !good_scale(q_descale) || !good_scale(k_descale) ||
      !good_scale(v_descale))
    return FA_ERR_UNSUPPORTED;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) ||
      !aligned(lse, 16))
    return FA_ERR_ALIGN;
  const size_t need = fa::fwd_split_workspace_bytes(B, H, N, d, causal ? 1 : 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return FA_ERR_ALIGN;
  fa::Fp8FwdArgs a{q8, k8, v8, q_descale, k_descale, v_descale, o, lse,
                   B, H, N, d, causal ? 1 : 0, softmax_scale};
  a.workspace = need > 0 ? workspace : nullptr;
  return fa::launch_fwd_fp8(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d, 2) != FA_OK) return 0;
  return fa::bwd_delta_bytes(B, H, N);
}

}  // extern "C"

namespace {

// Shape, workspace and alignment checks shared by the backward entry points.  `ptrs` are the tensor
// pointers the call uses (NULL ones were rejected before).
fa_status check_bwd(const void* const* ptrs, int n_ptrs, const void* workspace, size_t ws_bytes,
                    int B, int H, int N, int d, fa::BwdArgs* a) {
  fa_status st = check_shape(B, H, N, d, 2);
  if (st != FA_OK) return st;
  if (!workspace || ws_bytes < fa_bwd_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  for (int i = 0; i < n_ptrs; ++i)
    if (!aligned(ptrs[i], 16)) return FA_ERR_ALIGN;
  if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
  a->delta = (float*)workspace;
  a->B = B;
  a->H = H;
  a->N = N;
  a->d = d;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd_preprocess(const void* o, const void* dout, void* workspace,
                            size_t workspace_bytes, int B, int H, int N, int d,
                            hipStream_t stream) {
  if (!o || !dout) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {o, dout};
  fa_status st = check_bwd(ptrs, 2, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  a.o = o;
  a.dout = dout;
  return fa::launch_bwd_pre(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                      const void* dout, void* dk, void* dv, const void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d, int causal,
                      float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !lse || !dout || !dk || !dv) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {q, k, v, lse, dout, dk, dv};
  fa_status st = check_bwd(ptrs, 7, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.dout = dout;
  a.dk = dk;
  a.dv = dv;
  a.causal = causal ? 1 : 0;
  a.scale = a.dk_scale = a.dq_scale = softmax_scale;
  return fa::launch_bwd_dkdv(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, void* dq, const void* workspace, size_t workspace_bytes,
                    int B, int H, int N, int d, int causal, float softmax_scale,
                    hipStream_t stream) {
  if (!q || !k || !v || !lse || !dout || !dq) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {q, k, v, lse, dout, dq};
  fa_status st = check_bwd(ptrs, 6, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.causal = causal ? 1 : 0;
  a.scale = a.dk_scale = a.dq_scale = softmax_scale;
  return fa::launch_bwd_dq(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_delta_dq(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* workspace,
                          size_t workspace_bytes, int B, int H, int N, int d, int causal,
                          float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {q, k, v, o, lse, dout, dq};
  fa_status st = check_bwd(ptrs, 7, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.causal = causal ? 1 : 0;
  a.scale = a.dk_scale = a.dq_scale = softmax_scale;
  return fa::launch_bwd_delta_dq(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Shape checks of a decode call (everything fa_decode rejects before looking at pointers, scale
// and workspace).
fa_status check_decode_shape(int B, int H, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nq > 32 || Nk < Nq) return FA_ERR_SHAPE;
  fa_status st = check_shape(B, H, Nk, d, 2);  // the cache: per-head offsets, totals, grid
  if (st != FA_OK) return st;
  const fa::DecodeSplit sp = fa::decode_split(B, H, Nq, Nk);
  if ((uint64_t)B * (uint64_t)H * (uint64_t)sp.S >= (1ull << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (check_decode_shape(B, H, Nq, Nk, d) != FA_OK) return 0;
  return fa::decode_workspace_bytes(B, H, Nq, Nk, d);
}

fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                    int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_decode_shape(B, H, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa::decode_workspace_bytes(B, H, Nq, Nk, d))
    return FA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 16) || !aligned(workspace, 256))
    return FA_ERR_ALIGN;
  fa::DecodeArgs a{q, k, v, o, lse, workspace, B, H, Nq, Nk, d, causal ? 1 : 0, softmax_scale};
  return fa::launch_decode(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, int causal,
                 float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  fa_status st = check_bwd(ptrs, 9, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.causal = causal ? 1 : 0;
  a.scale = a.dk_scale = a.dq_scale = softmax_scale;
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_split_workspace_bytes(int B, int H, int N, int d, int causal) {
  if (check_shape(B, H, N, d, 2) != FA_OK) return 0;
  return fa::bwd_split_workspace_bytes(B, H, N, d, causal ? 1 : 0);
}

fa_status fa_bwd_split(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  fa_status st = check_bwd(ptrs, 9, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::bwd_split_workspace_bytes(B, H, N, d, causal ? 1 : 0))
    return FA_ERR_WORKSPACE;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.causal = causal ? 1 : 0;
  a.scale = a.dk_scale = a.dq_scale = softmax_scale;
  const fa::BwdSplit sp = fa::bwd_split(B, H, N, d, a.causal);
  if (sp.seg > 0) {  // partial sums after D: dQ's, then dK's and dV's
    char* p = (char*)workspace + fa::bwd_delta_bytes(B, H, N);
    a.split_seg = sp.seg;
    a.part_dq = (float*)p;
    p += fa::bwd_split_part_bytes(sp.nseg_q, B, H, N, d);
    a.part_dk = (float*)p;
    p += fa::bwd_split_part_bytes(sp.nseg_k, B, H, N, d);
    a.part_dv = (float*)p;
  }
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_fp8_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d, 2) != FA_OK) return 0;
  return fa::bwd_fp8_workspace_bytes(B, H, N, d);
}

fa_status fa_bwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale,
                     float k_descale, float v_descale, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, int causal,
                     float softmax_scale, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa::BwdArgs a{};
  const void* ptrs[] = {q8, k8, v8, o, lse, dout, dq, dk, dv};
  fa_status st = check_bwd(ptrs, 9, workspace, workspace_bytes, B, H, N, d, &a);
  if (st != FA_OK) return st;
  if (!good_scale(softmax_scale) || !good_scale(q_descale) || !good_scale(k_descale) ||
      !good_scale(v_descale))
    return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::bwd_fp8_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  // The scales must stay normal fp32 numbers once folded.
  const float score_scale = softmax_scale * q_descale * k_descale;
  const float dk_scale = softmax_scale * v_descale * q_descale;
  const float dq_scale = softmax_scale * v_descale * k_descale;
  const float delta_mult = 1.f / v_descale;
  if (!good_scale(score_scale) || !good_scale(dk_scale) || !good_scale(dq_scale) ||
      !good_scale(delta_mult) || !isnormal(score_scale) || !isnormal(dk_scale) ||
      !isnormal(dq_scale) || !isnormal(delta_mult))
    return FA_ERR_UNSUPPORTED;
  const size_t n = (size_t)B * H * N * d;
  char* ws = (char*)workspace;
  char* qc = ws + fa::bwd_delta_bytes(B, H, N);
  char* kc = qc + fa::bwd_fp8_image_bytes(B, H, N, d);
  char* vc = kc + fa::bwd_fp8_image_bytes(B, H, N, d);
  a.q = qc;
  a.k = kc;
  a.v = vc;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.causal = causal ? 1 : 0;
  a.scale = score_scale;
  a.dk_scale = dk_scale;
  a.dq_scale = dq_scale;
  a.delta_mult = delta_mult;
  if (fa::launch_e4m3_to_bf16(q8, qc, n, stream) != hipSuccess ||
      fa::launch_e4m3_to_bf16(k8, kc, n, stream) != hipSuccess ||
      fa::launch_e4m3_to_bf16(v8, vc, n, stream) != hipSuccess)
    return FA_ERR_LAUNCH;
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------------
// fa_bwd_noalloc: fa_bwd with its workspace (the fp32 D array) in a fixed device array of this
// library, for callers that cannot allocate.  Each device holds its own copy of `scratch` from the
// moment the library's code object is loaded on it until the process ends.  Host code never uses the
// array's name as a device address: the address of a device's copy is looked up once, with that
// device current, and kept per device.
namespace {

constexpr size_t kScratchRows = (size_t)1 << 22;  // D for B·H·N ≤ 2^22 rows: 16 MiB per device
static __device__ __align__(256) float scratch[kScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device; null until looked up

// Device address of `scratch` on the device `stream` belongs to.
fa_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream == nullptr) {
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_LAUNCH;
  } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    return FA_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_noalloc_max_rows(void) { return kScratchRows; }

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                         int H, int N, int d, int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, N, d, 2);
  if (st != FA_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N > (uint64_t)kScratchRows) return FA_ERR_WORKSPACE;
  if (!good_scale(softmax_scale)) return FA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return FA_ERR_ALIGN;
  void* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != FA_OK) return st;
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float*)ws;  // every row of D is written by the first kernel before the others read it
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.causal = causal ? 1 : 0;
  a.scale = a.dk_scale = a.dq_scale = softmax_scale;
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
