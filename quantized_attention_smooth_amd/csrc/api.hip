// C ABI of the gfx950 SageAttention2 forward (declared in include/sage_attn.h).
//
// Validation first, then the workspace is carved and the kernels are enqueued on the
// caller's stream.  Nothing is allocated, nothing is synchronised, no state is kept between
// calls (the last-error text is per thread).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/sage_attn.h"
#include "sage_internal.h"

// Workspace of sage_attn_fwd_noalloc: a file-scope device array, one copy on every GPU the library
// runs on, held until the process ends.  In host code `scratch` is only a stand-in for the symbol:
// its device address comes from hipGetSymbolAddress (per device, cached below) and only that
// address is ever passed to kernels.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return SAGE_ERR_HIP;
}

// Checks shared by every entry point; fills D (and, for varlen, the sequence table) on success.
int check_problem(const sage_problem_t* p, sage::Dims* D, std::vector<sage::Seq>* table) {
  if (p == nullptr) return SAGE_ERR_INVALID_ARG;
  if (p->cu_seqlens != nullptr && table == nullptr) return SAGE_ERR_INVALID_ARG;
  const int B = p->B, H = p->H, Hkv = p->Hkv, d = p->d;
  const bool varlen = p->cu_seqlens != nullptr;
  if (B < 1 || H < 1 || Hkv < 1 || (!varlen && p->N < 1)) return SAGE_ERR_INVALID_ARG;
  if (H % Hkv != 0) return SAGE_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return SAGE_ERR_INVALID_ARG;
  if (p->layout != SAGE_LAYOUT_HND && p->layout != SAGE_LAYOUT_NHD) return SAGE_ERR_INVALID_ARG;
  if (p->dtype != SAGE_DTYPE_FP16 && p->dtype != SAGE_DTYPE_BF16) return SAGE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (p->qk_bits != 4 && p->qk_bits != 8) return SAGE_ERR_UNSUPPORTED;
  if (p->pv_bits != 8 && p->pv_bits != 16) return SAGE_ERR_UNSUPPORTED;

  // per-sequence lengths: one N for all, or the differences of cu_seqlens
  long long nmax = 0, tot_pad = 0, tot_ds = 0, total = 0;
  if (varlen) {
    if (p->cu_seqlens[0] != 0) return SAGE_ERR_INVALID_ARG;
    table->resize(B);
  }
  for (int s = 0; s < B; ++s) {
    const long long n = varlen ? (long long)p->cu_seqlens[s + 1] - p->cu_seqlens[s] : p->N;
    if (n < 1) return SAGE_ERR_INVALID_ARG;
    if (n > (1 << 23)) return SAGE_ERR_UNSUPPORTED;   // exact fixed-point K sums need n <= 2^23
    const long long nb = (n + 127) / 128;
    if (varlen) {
      sage::Seq& e = (*table)[s];
      e.n = (int)n;
      e.tok0 = p->cu_seqlens[s];
      e.pad0 = (int)tot_pad;
      e.unused = 0;
      e.ds0 = tot_ds;
    }
    nmax = n > nmax ? n : nmax;
    total += n;
    tot_pad += nb * 128;
    tot_ds += (long long)H * (long long)sage::ds_head_elems(p->causal != 0, (int)nb, (int)(nb * 128));
    // every count the kernels index must fit comfortably in 64 bits; row offsets in 32 bits
    if (tot_pad > 2147483647LL || total > 2147483647LL) return SAGE_ERR_INVALID_ARG;
    if ((double)tot_pad * H * d > 9.0e18 || (double)tot_ds * 4.0 > 9.0e18) return SAGE_ERR_INVALID_ARG;
  }
  const long long npad = (nmax + 127) / 128 * 128;
  // 1-D grids: the statistics + Q prologue launch (128-token tiles of every kv head, then the Q
  // blocks of every head) is the largest; the attention launch (Q blocks of every head) and the
  // K/V codes + Delta_S launch (KV blocks of every kv head) are parts of it
  if ((double)B * H * (double)(npad / 128) + (double)B * Hkv * (double)((nmax + 127) / 128) > 2147483647.0)
    return SAGE_ERR_INVALID_ARG;
  D->B = B; D->H = H; D->Hkv = Hkv; D->N = (int)nmax; D->d = d; D->causal = p->causal;
  D->qk_bits = p->qk_bits; D->pv_bits = p->pv_bits;
  D->Npad = (int)npad;
  D->nqb = D->Npad / 128;
  D->nkb = D->Npad / 128;
  D->varlen = varlen ? 1 : 0;
  D->bf16 = p->dtype == SAGE_DTYPE_BF16 ? 1 : 0;
  D->tot_pad = tot_pad;
  D->tot_ds = tot_ds;
  // element strides (channels contiguous)
  sage::Strides& st = D->st;
  const long long N = nmax;
  if (varlen) {                        // packed [T, heads, d]
    st.qb = 0; st.qt = (long long)H * d; st.qh = d;
    st.kb = 0; st.kt = (long long)Hkv * d; st.kh = d;
  } else if (p->layout == SAGE_LAYOUT_HND) {   // [B, heads, N, d]
    st.qb = (long long)H * N * d; st.qt = d; st.qh = N * d;
    st.kb = (long long)Hkv * N * d; st.kt = d; st.kh = N * d;
  } else {                             // [B, N, heads, d]
    st.qb = N * H * d; st.qt = (long long)H * d; st.qh = d;
    st.kb = N * Hkv * d; st.kt = (long long)Hkv * d; st.kh = d;
  }
  return SAGE_OK;
}

sage_problem_t fixed_problem(int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits) {
  sage_problem_t p;
  memset(&p, 0, sizeof(p));
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N; p.d = d; p.causal = causal; p.qk_bits = qk_bits; p.pv_bits = pv_bits;
  p.layout = SAGE_LAYOUT_HND;
  p.dtype = SAGE_DTYPE_FP16;
  p.cu_seqlens = nullptr;
  return p;
}

int check_dims(int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits, sage::Dims* D) {
  const sage_problem_t p = fixed_problem(B, H, Hkv, N, d, causal, qk_bits, pv_bits);
  return check_problem(&p, D, nullptr);
}

int check_ws(void* ws, size_t ws_bytes, const sage::Layout& L) {
  if (ws == nullptr) return SAGE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % sage::WS_ALIGN != 0) return SAGE_ERR_WORKSPACE;
  if (ws_bytes < L.total) return SAGE_ERR_WORKSPACE;
  return SAGE_OK;
}

// What an entry point runs.
enum Work { kPrologue = 1, kAttend = 2, kBoth = 3 };

int run(const sage_problem_t* p, const void* q, const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
        void* stream, int work) {
  sage::Dims D;
  std::vector<sage::Seq> table;
  int st = check_problem(p, &D, &table);
  if (st != SAGE_OK) return st;
  const sage::Layout L = sage::make_layout(D);
  st = check_ws(ws, ws_bytes, L);
  if (st != SAGE_OK) return st;
  const sage::Ptrs P = sage::carve(ws, L, q, k, v, o);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (D.varlen) {
    e = sage::launch_seq_table(table.data(), D.B, P.seqs, s);
    if (e != hipSuccess) return hip_fail(e, "sequence table launch");
  }
  if (work & kPrologue) {
    e = sage::launch_prologue(D, P, s);
    if (e != hipSuccess) return hip_fail(e, "prologue launch");
  }
  if (work & kAttend) {
    e = sage::launch_attention(D, P, s);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
  }
  return SAGE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};      // device address of `scratch` on each device ordinal

// The device address of `scratch` on the current device, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_last_error, sizeof(g_last_error), "device ordinal %d beyond the %d the library tracks", dev, kMaxDevices);
    return SAGE_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % sage::WS_ALIGN != 0) {
      snprintf(g_last_error, sizeof(g_last_error), "scratch symbol address %p is not 256-byte aligned", ptr);
      return SAGE_ERR_HIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return SAGE_OK;
}

}  // namespace

extern "C" {

int sage_attn_fwd_noalloc(const sage_problem_t* p, const void* q, const void* k, const void* v, void* o,
                          void* stream) {
  if (!q || !k || !v || !o || p == nullptr) return SAGE_ERR_INVALID_ARG;
  if (p->cu_seqlens != nullptr) return SAGE_ERR_INVALID_ARG;      // fixed-length problems only
  sage::Dims D;
  int st = check_problem(p, &D, nullptr);
  if (st != SAGE_OK) return st;
  const size_t need = sage::make_layout(D).total;
  if (need > kScratchBytes) {
    snprintf(g_last_error, sizeof(g_last_error),
             "problem needs %zu bytes of workspace; the allocation-free entry point has %zu", need, kScratchBytes);
    return SAGE_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s != nullptr) {                      // the scratch copy used is the current device's
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != cur) {
      snprintf(g_last_error, sizeof(g_last_error), "stream is on device %d but device %d is current", sdev, cur);
      return SAGE_ERR_INVALID_ARG;
    }
  }
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SAGE_OK) return st;
  return run(p, q, k, v, o, ws, kScratchBytes, stream, kBoth);
}


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

int sage_attn_workspace_bytes_ex(const sage_problem_t* p, size_t* bytes) {
  if (bytes == nullptr) return SAGE_ERR_INVALID_ARG;
  sage::Dims D;
  std::vector<sage::Seq> table;
  const int st = check_problem(p, &D, &table);
  if (st != SAGE_OK) return st;
  *bytes = sage::make_layout(D).total;
  return SAGE_OK;
}

int sage_attn_fwd_ex(const sage_problem_t* p, const void* q, const void* k, const void* v, void* o,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return SAGE_ERR_INVALID_ARG;
  return run(p, q, k, v, o, workspace, workspace_bytes, stream, kBoth);
}

int sage_attn_prologue_ex(const sage_problem_t* p, const void* q, const void* k, const void* v, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !k || !v) return SAGE_ERR_INVALID_ARG;
  return run(p, q, k, v, nullptr, workspace, workspace_bytes, stream, kPrologue);
}

int sage_attn_attend_ex(const sage_problem_t* p, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  if (!o) return SAGE_ERR_INVALID_ARG;
  return run(p, nullptr, nullptr, nullptr, o, workspace, workspace_bytes, stream, kAttend);
}

int sage_attn_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits,
                              size_t* bytes) {
  const sage_problem_t p = fixed_problem(B, H, Hkv, N, d, causal, qk_bits, pv_bits);
  return sage_attn_workspace_bytes_ex(&p, bytes);
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Hkv, int N, int d,
                  int causal, int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes, void* stream) {
  const sage_problem_t p = fixed_problem(B, H, Hkv, N, d, causal, qk_bits, pv_bits);
  return sage_attn_fwd_ex(&p, q, k, v, o, workspace, workspace_bytes, stream);
}

int sage_attn_prologue(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N, int d,
                       int causal, int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const sage_problem_t p = fixed_problem(B, H, Hkv, N, d, causal, qk_bits, pv_bits);
  return sage_attn_prologue_ex(&p, q, k, v, workspace, workspace_bytes, stream);
}

int sage_attn_attend(void* o, int B, int H, int Hkv, int N, int d, int causal, int qk_bits, int pv_bits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const sage_problem_t p = fixed_problem(B, H, Hkv, N, d, causal, qk_bits, pv_bits);
  return sage_attn_attend_ex(&p, o, workspace, workspace_bytes, stream);
}

int sage_quant_debug_ex(const sage_problem_t* p, const void* q, const void* k, const void* v, void* workspace,
                        size_t workspace_bytes, void* stream, void* mu_k, void* k_codes, void* k_scales,
                        void* v_codes, void* v_scales, void* mu_q, void* q_codes, void* q_scales, void* delta_s) {
  if (!q || !k || !v || p == nullptr) return SAGE_ERR_INVALID_ARG;
  if (p->cu_seqlens != nullptr) return SAGE_ERR_INVALID_ARG;                  // fixed length only
  if (p->pv_bits == 16 && (v_codes || v_scales)) return SAGE_ERR_INVALID_ARG;   // V is not quantized
  sage::Dims D;
  int st = check_problem(p, &D, nullptr);
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

int sage_quant_debug(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N, int d, int causal,
                     int qk_bits, int pv_bits, void* workspace, size_t workspace_bytes, void* stream, void* mu_k,
                     void* k_codes, void* k_scales, void* v_codes, void* v_scales, void* mu_q, void* q_codes,
                     void* q_scales, void* delta_s) {
  const sage_problem_t p = fixed_problem(B, H, Hkv, N, d, causal, qk_bits, pv_bits);
  return sage_quant_debug_ex(&p, q, k, v, workspace, workspace_bytes, stream, mu_k, k_codes, k_scales, v_codes,
                             v_scales, mu_q, q_codes, q_scales, delta_s);
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
    case SAGE_ERR_INVALID_ARG:
      return "invalid argument (null pointer, size < 1, H % Hkv != 0, bad layout/dtype code, cu_seqlens not starting "
             "at 0 or not increasing, or size overflow)";
    case SAGE_ERR_UNSUPPORTED:
      return "unsupported configuration (d must be 64 or 128, qk_bits 4 or 8, pv_bits 8 or 16, sequence length <= 2^23)";
    case SAGE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case SAGE_ERR_HIP: return "HIP runtime error (see sage_last_error)";
    default: return "unknown status";
  }
}

const char* sage_last_error(void) { return g_last_error; }

int sage_mfma_rate_probe(int kind, int iters, void* sink, size_t sink_bytes, double* ops, void* stream) {
  if (kind < 0 || kind > 3 || iters < 1 || sink == nullptr || ops == nullptr) return SAGE_ERR_INVALID_ARG;
  if (sink_bytes < sage::mfma_probe_sink_bytes()) return SAGE_ERR_WORKSPACE;
  *ops = sage::mfma_probe_ops(kind, iters);
  const hipError_t e = sage::launch_mfma_probe(kind, iters, static_cast<float*>(sink), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return SAGE_OK;
}

}  // extern "C"
