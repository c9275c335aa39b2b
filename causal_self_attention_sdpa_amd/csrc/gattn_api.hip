// C-ABI entry points of libgattn: argument validation (before any HIP call)
// and dispatch to the float32 or 16-bit (bf16, fp16) kernels.  Semantics and error codes are
// documented in include/gattn.h.
#include "gattn.h"

#include <cmath>
#include <cstdint>
#include <mutex>

#include "gattn_internal.h"

// Device scratch of gattn_bwd_noalloc: the backward's row terms (what the
// caller's workspace holds for gattn_bwd), for callers that cannot allocate.
// Each GPU the library runs on holds its own copy for the life of the
// process.  In host code `scratch` is only a stand-in for the symbol: its
// device address comes from hipGetSymbolAddress (scratch_address below).
static constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using gattn::ws_part_bytes;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned(p, 16); }

int check_shape(int B, int H, int T, int hs, int dtype) {
  if (B < 1 || H < 1 || T < 1 || hs < 1) return GATTN_ERR_INVALID_ARG;
  if (dtype != GATTN_F32 && dtype != GATTN_BF16 && dtype != GATTN_F16) return GATTN_ERR_INVALID_ARG;
  if (int64_t(B) * H * T * hs >= (int64_t(1) << 31)) return GATTN_ERR_INVALID_ARG;
  // The 16-bit kernels address one (b, h) slice with 32-bit byte offsets and
  // touch rows up to the next tile boundary past T (fewer than 256 rows
  // further): those must still fit, as for the strided layouts (layout_of).
  if (dtype != GATTN_F32 && (int64_t(T) + 256) * hs * 2 >= (int64_t(1) << 31))
    return GATTN_ERR_INVALID_ARG;
  if (dtype != GATTN_F32 && hs != 32 && hs != 64) return GATTN_ERR_UNSUPPORTED;
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

// Strides {batch, head, row} in elements for a (B, H, T, hs) tensor with
// contiguous hs; nullptr means the contiguous layout.  Rows must not overlap
// (row stride >= hs), every row must start on a 16-byte boundary and the
// strides must be non-negative.  Kernels address a slice with 32-bit byte
// offsets and touch rows up to the next tile boundary past T (fewer than 256
// rows further), so T + 256 rows of the slice must span less than 2^31 bytes:
// a row past T then lies past the slice's range and reads as zero.
int layout_of(const int64_t* strides, int H, int T, int hs, int dtype, gattn::Layout& l) {
  if (strides == nullptr) {
    l = gattn::contiguous_layout(H, T, hs);
    return GATTN_OK;
  }
  const int64_t esize = dtype == GATTN_F32 ? 4 : 2;
  l = gattn::Layout{strides[0], strides[1], strides[2]};
  if (l.sb < 0 || l.sh < 0 || l.st < hs) return GATTN_ERR_INVALID_ARG;
  if ((l.sb * esize) % 16 || (l.sh * esize) % 16 || (l.st * esize) % 16) return GATTN_ERR_INVALID_ARG;
  if ((int64_t(T) + 256) * l.st * esize >= (int64_t(1) << 31)) return GATTN_ERR_INVALID_ARG;
  return GATTN_OK;
}

// Dropout parameters of probability p (finite, 0 <= p, rounding to a 16-bit
// threshold of at most 65535); thr = 0 (p rounds to 0) means no dropout.
int dropout_of(float p, uint64_t seed, uint32_t offset, gattn::Dropout& d) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return GATTN_ERR_INVALID_ARG;
  const double t = std::floor(double(p) * 65536.0 + 0.5);
  if (t > 65535.0) return GATTN_ERR_INVALID_ARG;
  d.thr = uint32_t(t);
  d.k0 = uint32_t(seed);
  d.k1 = uint32_t(seed >> 32);
  d.off = offset;
  d.zs = float(65536.0 / (65536.0 - t));
  d.izs = float((65536.0 - t) / 65536.0);
  d.lzs = float(std::log2(65536.0 / (65536.0 - t)));
  return GATTN_OK;
}

const gattn::Dropout kNoDropout{0, 0, 0, 0, 1.f, 1.f, 0.f};

// Workspace parts: D, then L2 = lse * log2(e).
float* ws_D(void* ws) { return static_cast<float*>(ws); }
float* ws_L2(void* ws, int B, int H, int T) {
  return reinterpret_cast<float*>(static_cast<char*>(ws) + ws_part_bytes(B, H, T));
}

// Implementations on layouts (arguments already validated).
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int T, int hs, float scale, int dtype, gattn::Layout li, gattn::Layout lo,
             const gattn::Dropout& dr, hipStream_t stream, void* keep = nullptr) {
  const int BH = B * H;
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_fwd(static_cast<const float*>(q), static_cast<const float*>(k),
                                    static_cast<const float*>(v), static_cast<float*>(o), lse, BH,
                                    H, T, T, hs, scale, li, li, lo, dr, stream));
  return status_of(gattn::h16_fwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                  static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                  static_cast<uint64_t*>(keep), BH, H, T, hs, scale, li, lo, dr,
                                  dtype == GATTN_F16, stream));
}

int pre_impl(const void* o, const void* dO, const float* lse, int B, int H, int T, int hs,
             int dtype, void* workspace, gattn::Layout lo, hipStream_t stream) {
  float* D = ws_D(workspace);
  float* L2 = ws_L2(workspace, B, H, T);
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_bwd_pre(static_cast<const float*>(o), static_cast<const float*>(dO),
                                        lse, D, L2, B * H, H, T, hs, lo, stream));
  return status_of(gattn::h16_bwd_pre(static_cast<const uint16_t*>(o),
                                      static_cast<const uint16_t*>(dO), lse, D, L2, B * H, H, T,
                                      hs, lo, dtype == GATTN_F16, stream));
}

// Keep-bit blocks of the 16-bit backward with dropout, after D and L2.
uint64_t* ws_keep(void* ws, int B, int H, int T) {
  return reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + 2 * ws_part_bytes(B, H, T));
}

// keep (dropout, 16-bit): NULL = the dQ pass draws the decisions and keeps
// them in the workspace; else the bits gattn_fwd_dropout stored.
int dq_impl(const void* q, const void* k, const void* v, const void* o, const void* dO,
            const float* lse, void* dq, int B, int H, int T, int hs, float scale, int dtype,
            void* workspace, gattn::Layout li, gattn::Layout lo, gattn::Layout lg,
            const gattn::Dropout& dr, hipStream_t stream, const void* keep = nullptr) {
  float* D = ws_D(workspace);
  float* L2 = ws_L2(workspace, B, H, T);
  if (dtype == GATTN_F32) {
    if (int st = pre_impl(o, dO, lse, B, H, T, hs, dtype, workspace, lo, stream)) return st;
    return status_of(gattn::f32_bwd_dq(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(dO), lse, D, static_cast<float*>(dq), B * H, H, T, hs, scale, li,
        lo, lg, dr, stream));
  }
  return status_of(gattn::h16_bwd_dq(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
      static_cast<const uint16_t*>(dO), lse, D, L2,
      dr.thr == 0 ? nullptr
                  : keep ? static_cast<uint64_t*>(const_cast<void*>(keep))
                         : ws_keep(workspace, B, H, T),
      keep != nullptr, static_cast<uint16_t*>(dq), B * H, H, T, hs, scale, li, lo, lg, dr,
      dtype == GATTN_F16, stream));
}

int dkdv_impl(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv,
              int B, int H, int T, int hs, float scale, int dtype, void* workspace,
              gattn::Layout li, gattn::Layout lo, gattn::Layout lg, const gattn::Dropout& dr,
              hipStream_t stream, const void* keep = nullptr) {
  const float* D = ws_D(workspace);
  const float* L2 = ws_L2(workspace, B, H, T);
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_bwd_dkdv(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(dO), D, L2, static_cast<float*>(dk), static_cast<float*>(dv),
        B * H, H, T, hs, scale, li, lo, lg, dr, stream));
  return status_of(gattn::h16_bwd_dkdv(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), D, L2,
      dr.thr == 0 ? nullptr
                  : keep ? static_cast<const uint64_t*>(keep) : ws_keep(workspace, B, H, T),
      static_cast<uint16_t*>(dk),
      static_cast<uint16_t*>(dv), B * H, H, T, hs, scale, li, lo, lg, dr, dtype == GATTN_F16,
      stream));
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              int B, int H, int T, int hs, float scale, int dtype) {
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 16)) return GATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return GATTN_ERR_INVALID_ARG;
  return check_shape(B, H, T, hs, dtype);
}

// Pointers, scale and shape of a backward call (everything but the workspace).
int check_bwd_io(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, const void* dq, const void* dk, const void* dv, int B, int H,
                 int T, int hs, float scale, int dtype) {
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(dO) || !ptr_ok(lse) ||
      !ptr_ok(dq) || !ptr_ok(dk) || !ptr_ok(dv))
    return GATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return GATTN_ERR_INVALID_ARG;
  return check_shape(B, H, T, hs, dtype);
}

int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, const void* dq, const void* dk, const void* dv, int B, int H,
              int T, int hs, float scale, int dtype, const void* ws, size_t wsb) {
  if (int st = check_bwd_io(q, k, v, o, dO, lse, dq, dk, dv, B, H, T, hs, scale, dtype))
    return st;
  return check_workspace(ws, wsb, B, H, T, hs, dtype);
}

// Device address of `scratch` on the current device, looked up with that
// device current the first time the device is seen and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GATTN_OK;
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

size_t gattn_dropout_keep_bytes(int B, int H, int T) {
  if (B < 1 || H < 1 || T < 1 || (int64_t(T) + 7) / 8 > gattn::kKeepMaxGroups) return 0;
  const int64_t ng = (int64_t(T) + 7) / 8;
  if (int64_t(B) * H > (int64_t(1) << 40) / (ng * ng * 8)) return 0;
  return gattn::ws_keep_bytes(B, H, T);
}

size_t gattn_bwd_dropout_workspace_bytes(int B, int H, int T, int hs, int dtype, float p) {
  gattn::Dropout dr;
  if (check_shape(B, H, T, hs, dtype) != GATTN_OK || dropout_of(p, 0, 0, dr) != GATTN_OK) return 0;
  const size_t base = 2 * ws_part_bytes(B, H, T);
  if (dtype == GATTN_F32 || dr.thr == 0) return base;
  if ((int64_t(T) + 7) / 8 > gattn::kKeepMaxGroups) return 0;
  return base + gattn::ws_keep_bytes(B, H, T);
}

int gattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int T, int hs, float scale, int dtype, hipStream_t stream) {
  if (int st = check_fwd(q, k, v, o, lse, B, H, T, hs, scale, dtype)) return st;
  const gattn::Layout c = gattn::contiguous_layout(H, T, hs);
  return fwd_impl(q, k, v, o, lse, B, H, T, hs, scale, dtype, c, c, kNoDropout, stream);
}

int gattn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int T, int hs, float scale, int dtype, const int64_t* qkv_strides,
                      const int64_t* o_strides, hipStream_t stream) {
  if (int st = check_fwd(q, k, v, o, lse, B, H, T, hs, scale, dtype)) return st;
  gattn::Layout li, lo;
  if (int st = layout_of(qkv_strides, H, T, hs, dtype, li)) return st;
  if (int st = layout_of(o_strides, H, T, hs, dtype, lo)) return st;
  return fwd_impl(q, k, v, o, lse, B, H, T, hs, scale, dtype, li, lo, kNoDropout, stream);
}

int gattn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int T, int hs, float scale, int dtype, float p, uint64_t seed,
                      uint32_t offset, void* keep, const int64_t* qkv_strides,
                      const int64_t* o_strides, hipStream_t stream) {
  if (int st = check_fwd(q, k, v, o, lse, B, H, T, hs, scale, dtype)) return st;
  gattn::Dropout dr;
  if (int st = dropout_of(p, seed, offset, dr)) return st;
  if (keep != nullptr && (!aligned(keep, 16) || gattn_dropout_keep_bytes(B, H, T) == 0))
    return GATTN_ERR_INVALID_ARG;
  gattn::Layout li, lo;
  if (int st = layout_of(qkv_strides, H, T, hs, dtype, li)) return st;
  if (int st = layout_of(o_strides, H, T, hs, dtype, lo)) return st;
  return fwd_impl(q, k, v, o, lse, B, H, T, hs, scale, dtype, li, lo, dr, stream, keep);
}

int gattn_probe_mfma_bf16(float* sink, int blocks, int iters, hipStream_t stream) {
  if (sink == nullptr || blocks < 1 || iters < 1) return GATTN_ERR_INVALID_ARG;
  return status_of(gattn::mfma_loop(sink, blocks, iters, stream));
}

int gattn_probe_issue(float* sink, int blocks, int mfma_iters, int valu_iters, int kind,
                      int roles, hipStream_t stream) {
  if (sink == nullptr || blocks < 1 || mfma_iters < 0 || valu_iters < 0 || kind < 0 || kind > 2 ||
      roles < 1 || roles > 15)
    return GATTN_ERR_INVALID_ARG;
  return status_of(gattn::issue_probe(sink, blocks, mfma_iters, valu_iters, kind, roles, stream));
}

int gattn_dropout_mask(uint8_t* keep, int B, int H, int T, float p, uint64_t seed,
                       uint32_t offset, hipStream_t stream) {
  if (keep == nullptr || B < 1 || H < 1 || T < 1) return GATTN_ERR_INVALID_ARG;
  if (int64_t(B) * H * T * T >= (int64_t(1) << 40) || int64_t(B) * H >= (int64_t(1) << 31))
    return GATTN_ERR_INVALID_ARG;
  gattn::Dropout dr;
  if (int st = dropout_of(p, seed, offset, dr)) return st;
  return status_of(gattn::dropout_mask(keep, B * H, T, dr, stream));
}

size_t gattn_fwd_decode_workspace_bytes(int B, int H, int Tq, int Tk, int hs, int dtype) {
  if (Tk < Tq || check_shape(B, H, Tk, hs, dtype) != GATTN_OK) return 0;
  if (dtype == GATTN_F32) return 0;
  const gattn::DecodeSplit d = gattn::decode_split(B * H, Tq, Tk);
  if (d.nsplit == 1) return 0;  // one split: the result is written directly
  return gattn::decode_opart_bytes(B * H, Tq, hs, d) + gattn::decode_lpart_bytes(B * H, Tq, d);
}

int gattn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Tq, int Tk, int hs, float scale, int dtype,
                     const int64_t* q_strides, const int64_t* kv_strides,
                     const int64_t* o_strides, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 16)) return GATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return GATTN_ERR_INVALID_ARG;
  if (Tq < 1 || Tk < Tq) return GATTN_ERR_INVALID_ARG;
  if (int st = check_shape(B, H, Tk, hs, dtype)) return st;
  gattn::Layout lq, lk, lo;
  if (int st = layout_of(q_strides, H, Tq, hs, dtype, lq)) return st;
  if (int st = layout_of(kv_strides, H, Tk, hs, dtype, lk)) return st;
  if (int st = layout_of(o_strides, H, Tq, hs, dtype, lo)) return st;
  const int BH = B * H;
  if (dtype == GATTN_F32)
    return status_of(gattn::f32_fwd(static_cast<const float*>(q), static_cast<const float*>(k),
                                    static_cast<const float*>(v), static_cast<float*>(o), lse, BH,
                                    H, Tq, Tk, hs, scale, lq, lk, lo, kNoDropout, stream));
  const size_t need = gattn_fwd_decode_workspace_bytes(B, H, Tq, Tk, hs, dtype);
  if (need > 0 && (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need))
    return GATTN_ERR_WORKSPACE;
  const gattn::DecodeSplit d = gattn::decode_split(BH, Tq, Tk);
  float* opart = static_cast<float*>(workspace);
  float* lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          gattn::decode_opart_bytes(BH, Tq, hs, d));
  return status_of(gattn::h16_fwd_decode(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH, H, Tq, Tk, hs, scale,
      lq, lk, lo, opart, lpart, d, dtype == GATTN_F16, stream));
}

int gattn_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int T,
                         int hs, int dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!ptr_ok(o) || !ptr_ok(dO) || !ptr_ok(lse)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_shape(B, H, T, hs, dtype)) return st;
  if (int st = check_workspace(workspace, workspace_bytes, B, H, T, hs, dtype)) return st;
  return pre_impl(o, dO, lse, B, H, T, hs, dtype, workspace, gattn::contiguous_layout(H, T, hs),
                  stream);
}

int gattn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, void* dq, int B, int H, int T, int hs, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(dq)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_main(q, k, v, dO, scale, B, H, T, hs, dtype, workspace, workspace_bytes))
    return st;
  const gattn::Layout c = gattn::contiguous_layout(H, T, hs);
  return dq_impl(q, k, v, o, dO, lse, dq, B, H, T, hs, scale, dtype, workspace, c, c, c,
                 kNoDropout, stream);
}

int gattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, void* dk,
                   void* dv, int B, int H, int T, int hs, float scale, int dtype, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  if (!ptr_ok(dk) || !ptr_ok(dv)) return GATTN_ERR_INVALID_ARG;
  if (int st = check_main(q, k, v, dO, scale, B, H, T, hs, dtype, workspace, workspace_bytes))
    return st;
  const gattn::Layout c = gattn::contiguous_layout(H, T, hs);
  return dkdv_impl(q, k, v, dO, dk, dv, B, H, T, hs, scale, dtype, workspace, c, c, c,
                   kNoDropout, stream);
}

int gattn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int hs,
              float scale, int dtype, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  // Validate everything up front so that a rejected call enqueues nothing.
  if (int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, T, hs, scale, dtype, workspace,
                         workspace_bytes))
    return st;
  const gattn::Layout c = gattn::contiguous_layout(H, T, hs);
  if (int st = dq_impl(q, k, v, o, dO, lse, dq, B, H, T, hs, scale, dtype, workspace, c, c, c,
                       kNoDropout, stream))
    return st;
  return dkdv_impl(q, k, v, dO, dk, dv, B, H, T, hs, scale, dtype, workspace, c, c, c, kNoDropout,
                   stream);
}

size_t gattn_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

int gattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int hs,
                      float scale, int dtype, hipStream_t stream) {
  if (int st = check_bwd_io(q, k, v, o, dO, lse, dq, dk, dv, B, H, T, hs, scale, dtype))
    return st;
  if (gattn_bwd_workspace_bytes(B, H, T, hs, dtype) > kScratchBytes) return GATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (int st = scratch_address(&ws)) return st;
  // The row terms need no clearing: the dQ pass (or, for float32, the row
  // pass) overwrites every one the dK/dV pass reads.
  const gattn::Layout c = gattn::contiguous_layout(H, T, hs);
  if (int st = dq_impl(q, k, v, o, dO, lse, dq, B, H, T, hs, scale, dtype, ws, c, c, c,
                       kNoDropout, stream))
    return st;
  return dkdv_impl(q, k, v, dO, dk, dv, B, H, T, hs, scale, dtype, ws, c, c, c, kNoDropout,
                   stream);
}

int gattn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int hs,
                      float scale, int dtype, void* workspace, size_t workspace_bytes,
                      const int64_t* qkv_strides, const int64_t* o_strides,
                      const int64_t* grad_strides, hipStream_t stream) {
  if (int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, T, hs, scale, dtype, workspace,
                         workspace_bytes))
    return st;
  gattn::Layout li, lo, lg;
  if (int st = layout_of(qkv_strides, H, T, hs, dtype, li)) return st;
  if (int st = layout_of(o_strides, H, T, hs, dtype, lo)) return st;
  if (int st = layout_of(grad_strides, H, T, hs, dtype, lg)) return st;
  if (int st = dq_impl(q, k, v, o, dO, lse, dq, B, H, T, hs, scale, dtype, workspace, li, lo, lg,
                       kNoDropout, stream))
    return st;
  return dkdv_impl(q, k, v, dO, dk, dv, B, H, T, hs, scale, dtype, workspace, li, lo, lg,
                   kNoDropout, stream);
}

int gattn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int hs,
                      float scale, int dtype, float p, uint64_t seed, uint32_t offset,
                      const void* keep, void* workspace, size_t workspace_bytes,
                      const int64_t* qkv_strides, const int64_t* o_strides,
                      const int64_t* grad_strides, hipStream_t stream) {
  if (int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, T, hs, scale, dtype, workspace,
                         workspace_bytes))
    return st;
  gattn::Dropout dr;
  if (int st = dropout_of(p, seed, offset, dr)) return st;
  if (dtype != GATTN_F32 && dr.thr != 0 && (int64_t(T) + 7) / 8 > gattn::kKeepMaxGroups)
    return GATTN_ERR_INVALID_ARG;
  if (keep != nullptr && (!aligned(keep, 16) || gattn_dropout_keep_bytes(B, H, T) == 0))
    return GATTN_ERR_INVALID_ARG;
  if (dtype == GATTN_F32 || dr.thr == 0) keep = nullptr;  // the float32 path draws its own
  if (keep == nullptr &&
      workspace_bytes < gattn_bwd_dropout_workspace_bytes(B, H, T, hs, dtype, p))
    return GATTN_ERR_WORKSPACE;
  gattn::Layout li, lo, lg;
  if (int st = layout_of(qkv_strides, H, T, hs, dtype, li)) return st;
  if (int st = layout_of(o_strides, H, T, hs, dtype, lo)) return st;
  if (int st = layout_of(grad_strides, H, T, hs, dtype, lg)) return st;
  if (int st = dq_impl(q, k, v, o, dO, lse, dq, B, H, T, hs, scale, dtype, workspace, li, lo, lg,
                       dr, stream, keep))
    return st;
  return dkdv_impl(q, k, v, dO, dk, dv, B, H, T, hs, scale, dtype, workspace, li, lo, lg, dr,
                   stream, keep);
}

}  // extern "C"
