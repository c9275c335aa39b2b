// C-ABI entry points of libgattn: argument validation (before any HIP call)
// and dispatch to the float32 or bf16 kernels.  Semantics and error codes are
// documented in include/gattn.h.
#include "gattn.h"

#include <cmath>
#include <cstdint>

#include "gattn_internal.h"

namespace {

using gattn::ws_part_bytes;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned(p, 16); }

int check_shape(int B, int H, int T, int hs, int dtype) {
  if (B < 1 || H < 1 || T < 1 || hs < 1) return GATTN_ERR_INVALID_ARG;
  if (dtype != GATTN_F32 && dtype != GATTN_BF16) return GATTN_ERR_INVALID_ARG;
  if (int64_t(B) * H * T * hs >= (int64_t(1) << 31)) return GATTN_ERR_INVALID_ARG;
  if (dtype == GATTN_BF16 && hs != 32 && hs != 64) return GATTN_ERR_UNSUPPORTED;
  if (dtype == GATTN_F32 && hs > 128) return GATTN_ERR_UNSUPPORTED;
  return GATTN_OK;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

int check_workspace(const void* ws, size_t bytes, int B, int H, int T, int hs, int dtype) {
  if (ws == nullptr || !aligned(ws, 256)) return GATTN_ERR_WORKSPACE;
  if (bytes < gattn_bwd_workspace_bytes(B, H, T, hs, dtype)) return GATTN_ERR_WORKSPACE;
  return GATTN_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? GATTN_OK : GATTN_ERR_HIP; }

// Checks shared by the two main backward stages.
int check_main(const void* q, const void* k, const void* v, const void* dO, float scale, int B,
               int H, int T, int hs, int dtype, const void* ws, size_t wsb) {
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(dO)) return GATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_shape(B, H, T, hs, dtype)) return st;
  return check_workspace(ws, wsb, B, H, T, hs, dtype);
}

// Workspace parts: D, then L2 = lse * log2(e).
float* ws_D(void* ws) { return static_cast<float*>(ws); }
float* ws_L2(void* ws, int B, int H, int T) {
  return reinterpret_cast<float*>(static_cast<char*>(ws) + ws_part_bytes(B, H, T));
}

}  // namespace

extern "C" {

const char* gattn_status_string(int status) {
  switch (status) {
    case GATTN_OK: return "GATTN_OK";
    case GATTN_ERR_INVALID_ARG: return "GATTN_ERR_INVALID_ARG";
    case GATTN_ERR_UNSUPPORTED: return "GATTN_ERR_UNSUPPORTED";
    case GATTN_ERR_WORKSPACE: return "GATTN_ERR_WORKSPACE";
    case GATTN_ERR_HIP: return "GATTN_ERR_HIP";
    default: return "GATTN_UNKNOWN_STATUS";
  }
}

size_t gattn_bwd_workspace_bytes(int B, int H, int T, int hs, int dtype) {
  if (check_shape(B, H, T, hs, dtype) != GATTN_OK) return 0;
  return 2 * ws_part_bytes(B, H, T);
}

int gattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int T, int hs, float scale, int dtype, hipStream_t stream) {
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 16)) return GATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_shape(B, H, T, hs, dtype)) return st;
  const int BH = B * H;
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_fwd(static_cast<const float*>(q), static_cast<const float*>(k),
                                    static_cast<const float*>(v), static_cast<float*>(o), lse, BH,
                                    T, hs, scale, stream));
  return status_of(gattn::bf16_fwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                   static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                   BH, T, hs, scale, stream));
}

int gattn_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int T,
                         int hs, int dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!ptr_ok(o) || !ptr_ok(dO) || !ptr_ok(lse)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_shape(B, H, T, hs, dtype)) return st;
  if (int st = check_workspace(workspace, workspace_bytes, B, H, T, hs, dtype)) return st;
  float* D = ws_D(workspace);
  float* L2 = ws_L2(workspace, B, H, T);
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_bwd_pre(static_cast<const float*>(o), static_cast<const float*>(dO),
                                        lse, D, L2, B * H, T, hs, stream));
  return status_of(gattn::bf16_bwd_pre(static_cast<const uint16_t*>(o),
                                       static_cast<const uint16_t*>(dO), lse, D, L2, B * H, T, hs,
                                       stream));
}

int gattn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, void* dq, int B, int H, int T, int hs, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(dq)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_main(q, k, v, dO, scale, B, H, T, hs, dtype, workspace, workspace_bytes))
    return st;
  float* D = ws_D(workspace);
  float* L2 = ws_L2(workspace, B, H, T);
  if (dtype == GATTN_F32) {
    hipError_t e = gattn::f32_bwd_pre(static_cast<const float*>(o), static_cast<const float*>(dO),
                                      lse, D, L2, B * H, T, hs, stream);
    if (e != hipSuccess) return GATTN_ERR_HIP;
    return status_of(gattn::f32_bwd_dq(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(dO), lse, D, static_cast<float*>(dq), B * H, T, hs, scale,
        stream));
  }
  return status_of(gattn::bf16_bwd_dq(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
      static_cast<const uint16_t*>(dO), lse, D, L2, static_cast<uint16_t*>(dq), B * H, T, hs,
      scale, stream));
}

int gattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, void* dk,
                   void* dv, int B, int H, int T, int hs, float scale, int dtype, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  if (!ptr_ok(dk) || !ptr_ok(dv)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_main(q, k, v, dO, scale, B, H, T, hs, dtype, workspace, workspace_bytes))
    return st;
  const float* D = ws_D(workspace);
  const float* L2 = ws_L2(workspace, B, H, T);
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_bwd_dkdv(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(dO), D, L2, static_cast<float*>(dk), static_cast<float*>(dv),
        B * H, T, hs, scale, stream));
  return status_of(gattn::bf16_bwd_dkdv(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), D, L2,
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), B * H, T, hs, scale, stream));
}

int gattn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int hs,
              float scale, int dtype, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  // Validate everything up front so that a rejected call enqueues nothing.
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(dO) || !ptr_ok(lse) ||
      !ptr_ok(dq) || !ptr_ok(dk) || !ptr_ok(dv))
    return GATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_shape(B, H, T, hs, dtype)) return st;
  if (int st = check_workspace(workspace, workspace_bytes, B, H, T, hs, dtype)) return st;
  int st = gattn_bwd_dq(q, k, v, o, dO, lse, dq, B, H, T, hs, scale, dtype, workspace,
                        workspace_bytes, stream);
  if (st != GATTN_OK) return st;
  return gattn_bwd_dkdv(q, k, v, dO, dk, dv, B, H, T, hs, scale, dtype, workspace, workspace_bytes,
                        stream);
}

}  // extern "C"
