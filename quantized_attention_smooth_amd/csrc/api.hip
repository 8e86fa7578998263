// C ABI of the gfx950 SageAttention2 forward (declared in include/sage_attn.h).
//
// Validation first, then the workspace is carved and the kernels are enqueued on the
// caller's stream.  Nothing is allocated, nothing is synchronised, no state is kept between
// calls (the last-error text is per thread).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/sage_attn.h"
#include "sage_internal.h"

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return SAGE_ERR_HIP;
}

// Shape checks shared by every entry point; fills D on success.
int check_dims(int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits, sage::Dims* D) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (H % Hkv != 0) return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (qk_bits != 4 && qk_bits != 8) return SAGE_ERR_UNSUPPORTED;
  if (pv_bits != 8 && pv_bits != 16) return SAGE_ERR_UNSUPPORTED;
  if (N > (1 << 23)) return SAGE_ERR_UNSUPPORTED;   // exact fixed-point K sums need N <= 2^23
  const long long npad = ((long long)N + 127) / 128 * 128;
  // every element count the kernels index must fit comfortably in 64 bits, and the number of
  // workgroups in a 1-D grid must fit in 32 bits
  const double heads = (double)B * (double)H;
  if (heads * (double)npad * (double)d > 9.0e18) return SAGE_ERR_INVALID_ARG;
  if (heads * (double)(npad / 128) * (double)npad * 4.0 > 9.0e18) return SAGE_ERR_INVALID_ARG;
  if (heads * (double)(npad / 128) > 2147483647.0) return SAGE_ERR_INVALID_ARG;
  if ((double)B * Hkv > 65535.0 || heads > 65535.0) return SAGE_ERR_INVALID_ARG;   // grid.y/z limits
  D->B = B; D->H = H; D->Hkv = Hkv; D->N = N; D->d = d; D->causal = causal; D->qk_bits = qk_bits; D->pv_bits = pv_bits;
  D->Npad = (int)npad;
  D->nqb = D->Npad / 128;
  D->nkb = D->Npad / 128;
  return SAGE_OK;
}

int check_ws(void* ws, size_t ws_bytes, const sage::Layout& L) {
  if (ws == nullptr) return SAGE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % sage::WS_ALIGN != 0) return SAGE_ERR_WORKSPACE;
  if (ws_bytes < L.total) return SAGE_ERR_WORKSPACE;
  return SAGE_OK;
}

}  // namespace

extern "C" {

int sage_get_config(sage_config_t* out) {
  if (out == nullptr) return SAGE_ERR_INVALID_ARG;
  out->version = 1;
  out->bq = sage::BQ;
  out->bk = sage::BK;
  out->q_slice = 1;
  out->q_period = 1;
  out->q_run = 1;
  out->k_slice = sage::BK;
  out->k_period = 8;
  out->k_run = 4;
  out->p_range = sage::P_RANGE;
  out->v_range = sage::V_RANGE;
  out->fp8_format = 1;
  return SAGE_OK;
}

int sage_attn_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits,
                              size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_INVALID_ARG;
  sage::Dims D;
  const int st = check_dims(B, H, Hkv, N, d, causal, qk_bits, pv_bits, &D);
  if (st != SAGE_OK) return st;
  *bytes = sage::make_layout(D).total;
  return SAGE_OK;
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Hkv, int N, int d,
                  int causal, int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return SAGE_ERR_INVALID_ARG;
  sage::Dims D;
  int st = check_dims(B, H, Hkv, N, d, causal, qk_bits, pv_bits, &D);
  if (st != SAGE_OK) return st;
  const sage::Layout L = sage::make_layout(D);
  st = check_ws(workspace, workspace_bytes, L);
  if (st != SAGE_OK) return st;
  const sage::Ptrs P = sage::carve(workspace, L, q, k, v, o);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sage::launch_prologue(D, P, s);
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  e = sage::launch_attention(D, P, s);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return SAGE_OK;
}

int sage_attn_prologue(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N, int d,
                       int causal, int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!q || !k || !v) return SAGE_ERR_INVALID_ARG;
  sage::Dims D;
  int st = check_dims(B, H, Hkv, N, d, causal, qk_bits, pv_bits, &D);
  if (st != SAGE_OK) return st;
  const sage::Layout L = sage::make_layout(D);
  st = check_ws(workspace, workspace_bytes, L);
  if (st != SAGE_OK) return st;
  const sage::Ptrs P = sage::carve(workspace, L, q, k, v, nullptr);
  const hipError_t e = sage::launch_prologue(D, P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAGE_OK : hip_fail(e, "prologue launch");
}

int sage_attn_attend(void* o, int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!o) return SAGE_ERR_INVALID_ARG;
  sage::Dims D;
  int st = check_dims(B, H, Hkv, N, d, causal, qk_bits, pv_bits, &D);
  if (st != SAGE_OK) return st;
  const sage::Layout L = sage::make_layout(D);
  st = check_ws(workspace, workspace_bytes, L);
  if (st != SAGE_OK) return st;
  const sage::Ptrs P = sage::carve(workspace, L, nullptr, nullptr, nullptr, o);
  const hipError_t e = sage::launch_attention(D, P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAGE_OK : hip_fail(e, "attention launch");
}

int sage_quant_debug(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N, int d, int causal,
                     int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes, void* stream, void* mu_k,
                     void* k_codes, void* k_scales, void* v_codes, void* v_scales, void* mu_q, void* q_codes,
                     void* q_scales, void* delta_s) {
  if (!q || !k || !v) return SAGE_ERR_INVALID_ARG;
  if (pv_bits == 16 && (v_codes || v_scales)) return SAGE_ERR_INVALID_ARG;   // V is not quantized
  sage::Dims D;
  int st = check_dims(B, H, Hkv, N, d, causal, qk_bits, pv_bits, &D);
  if (st != SAGE_OK) return st;
  const sage::Layout L = sage::make_layout(D);
  st = check_ws(workspace, workspace_bytes, L);
  if (st != SAGE_OK) return st;
  const sage::Ptrs P = sage::carve(workspace, L, q, k, v, nullptr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sage::launch_prologue(D, P, s);
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  e = sage::launch_debug_copy(D, P, s, static_cast<float*>(mu_k), static_cast<int8_t*>(k_codes),
                              static_cast<float*>(k_scales), static_cast<uint8_t*>(v_codes),
                              static_cast<float*>(v_scales), static_cast<float*>(mu_q),
                              static_cast<int8_t*>(q_codes), static_cast<float*>(q_scales),
                              static_cast<float*>(delta_s));
  if (e != hipSuccess) return hip_fail(e, "debug copy");
  return SAGE_OK;
}

int sage_qk_tile_debug(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N, int d, int causal,
                       int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes, void* stream, int b, int h,
                       int qb, int kb, int32_t* tile_out) {
  if (!q || !k || !v || !tile_out) return SAGE_ERR_INVALID_ARG;
  sage::Dims D;
  int st = check_dims(B, H, Hkv, N, d, causal, qk_bits, pv_bits, &D);
  if (st != SAGE_OK) return st;
  if (b < 0 || b >= B || h < 0 || h >= H || qb < 0 || qb >= D.nqb || kb < 0 || kb >= D.nkb)
    return SAGE_ERR_INVALID_ARG;
  const sage::Layout L = sage::make_layout(D);
  st = check_ws(workspace, workspace_bytes, L);
  if (st != SAGE_OK) return st;
  const sage::Ptrs P = sage::carve(workspace, L, q, k, v, nullptr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sage::launch_prologue(D, P, s);
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  e = sage::launch_qk_tile(D, P, b, h, qb, kb, tile_out, s);
  if (e != hipSuccess) return hip_fail(e, "qk tile launch");
  return SAGE_OK;
}

const char* sage_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_INVALID_ARG: return "invalid argument (null pointer, size < 1, H % Hkv != 0 or size overflow)";
    case SAGE_ERR_UNSUPPORTED: return "unsupported configuration (d must be 64 or 128, qk_bits 4 or 8, pv_bits 8 or 16, N <= 2^23)";
    case SAGE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case SAGE_ERR_HIP: return "HIP runtime error (see sage_last_error)";
    default: return "unknown status";
  }
}

const char* sage_last_error(void) { return g_last_error; }

}  // extern "C"
