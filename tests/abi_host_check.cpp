// Host-side check of the C ABI's argument validation, workspace carve-up and varlen sequence
// table, built from the library's own host source (csrc/api.hip) with AddressSanitizer and
// UndefinedBehaviorSanitizer and run without a GPU.
//
// The kernel launchers are replaced by stand-ins that touch, in ordinary host memory, every
// byte of every workspace section the kernels use, with the extents the layout documents
// (csrc/sage_internal.h), and every byte of the output tensor: a section that the carve-up
// places outside the workspace, or a workspace-size computation that falls short, makes
// AddressSanitizer stop the program; signed overflow in the validation arithmetic makes
// UndefinedBehaviorSanitizer stop it.  Prints "ok" when every case passes.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../include/sage_attn.h"
#include "../quantized_attention_smooth_amd/csrc/sage_internal.h"

namespace {
int g_fail = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      g_fail = 1;                                                    \
    }                                                                \
  } while (0)

volatile unsigned char g_sink;
void touch(const void* p, size_t n) {         // read every byte and write it back unchanged
  volatile unsigned char* b = (volatile unsigned char*)const_cast<void*>(p);
  unsigned char acc = 0;
  for (size_t i = 0; i < n; ++i) { const unsigned char x = b[i]; acc ^= x; b[i] = x; }
  g_sink = acc;
}

size_t g_o_bytes = 0;                          // output bytes of the current case
const sage::Seq* g_table_seen = nullptr;
}  // namespace

namespace sage {
hipError_t launch_seq_table(const Seq* host, int n, Seq* dev, hipStream_t) {
  memcpy(dev, host, (size_t)n * sizeof(Seq));
  g_table_seen = dev;
  return hipSuccess;
}
// Every section the prologue writes, with its documented extent: each is filled with its own
// tag byte and checked afterwards, so sections that overlap (or run past the workspace, which
// AddressSanitizer reports) are found.  The sequence table is only read.
hipError_t launch_prologue(const Dims& D, const Ptrs& P, hipStream_t) {
  const size_t B = D.B, H = D.H, Hkv = D.Hkv, T = (size_t)D.tot_pad, d = D.d, nb = T / BQ;
  struct Sec { void* p; size_t n; };
  const Sec secs[] = {
      {P.kcodes, Hkv * T * d}, {P.vcodes, Hkv * T * d * (D.pv_bits / 8)}, {P.qcodes, H * T * d},
      {P.kscale, Hkv * nb * 2 * 4}, {P.qscale, H * T * 4}, {P.muk, B * Hkv * d * 4},
      {P.ksum, B * Hkv * d * 8 * (D.bf16 ? 12 : 1)}, {P.vamax, B * Hkv * d * 4}, {P.vscale, B * Hkv * d * 4},
      {P.muq, H * nb * d * 4}, {P.muqs, H * nb * 3 * d * 2}, {P.ds, (size_t)D.tot_ds * 4}};
  const int ns = (int)(sizeof(secs) / sizeof(secs[0]));
  for (int i = 0; i < ns; ++i) memset(secs[i].p, 0x40 + i, secs[i].n);
  for (int i = 0; i < ns; ++i) {
    const unsigned char* b = static_cast<const unsigned char*>(secs[i].p);
    size_t bad = 0;
    for (size_t j = 0; j < secs[i].n; ++j) bad += b[j] != 0x40 + i;
    CHECK(bad == 0);
  }
  if (D.varlen) touch(P.seqs, B * sizeof(Seq));
  return hipSuccess;
}
hipError_t launch_attention(const Dims&, const Ptrs& P, hipStream_t) {
  touch(P.o, g_o_bytes);
  return hipSuccess;
}
hipError_t launch_qk_tile(const Dims&, const Ptrs&, int, int, int, int, int32_t* out, hipStream_t) {
  touch(out, (size_t)BQ * BK * 4);
  return hipSuccess;
}
hipError_t launch_debug_copy(const Dims&, const Ptrs&, hipStream_t, float*, int8_t*, float*, uint8_t*, float*,
                             float*, int8_t*, float*, float*) {
  return hipSuccess;
}
double mfma_probe_ops(int, int iters) { return 1.0 * iters; }
size_t mfma_probe_sink_bytes() { return 512 * 1024; }
hipError_t launch_mfma_probe(int, int, float* sink, hipStream_t) {
  touch(sink, mfma_probe_sink_bytes());
  return hipSuccess;
}
}  // namespace sage

namespace {
// one full call on host buffers of exactly the sizes the ABI promises
void run_case(const sage_problem_t& p) {
  size_t ws_bytes = 0;
  CHECK(sage_attn_workspace_bytes_ex(&p, &ws_bytes) == SAGE_OK);
  const long long T = p.cu_seqlens ? p.cu_seqlens[p.B] : (long long)p.B * p.N;
  const size_t es = 2;                                 // fp16 / bf16
  const size_t qbytes = (size_t)T * p.H * p.d * es, kbytes = (size_t)T * p.Hkv * p.d * es;
  void* ws = aligned_alloc(256, (ws_bytes + 255) / 256 * 256);
  void* q = malloc(qbytes);
  void* k = malloc(kbytes);
  void* v = malloc(kbytes);
  void* o = malloc(qbytes);
  memset(ws, 0, ws_bytes);
  g_o_bytes = qbytes;
  g_table_seen = nullptr;
  CHECK(sage_attn_fwd_ex(&p, q, k, v, o, ws, ws_bytes, nullptr) == SAGE_OK);
  if (p.cu_seqlens) {
    CHECK(g_table_seen != nullptr);
    // the table the kernels read: lengths, token offsets, padded rows, Delta_S offsets
    long long pad = 0, ds = 0;
    for (int s = 0; s < p.B && g_table_seen; ++s) {
      const sage::Seq& e = g_table_seen[s];
      const int n = p.cu_seqlens[s + 1] - p.cu_seqlens[s];
      CHECK(e.n == n && e.tok0 == p.cu_seqlens[s] && e.pad0 == pad && e.ds0 == ds);
      const int nbs = (n + 127) / 128;
      pad += 128LL * nbs;
      ds += (long long)p.H * (long long)sage::ds_head_elems(p.causal != 0, nbs, nbs * 128);
    }
  }
  // one byte short of the workspace is rejected before anything runs
  CHECK(sage_attn_fwd_ex(&p, q, k, v, o, ws, ws_bytes - 1, nullptr) == SAGE_ERR_WORKSPACE);
  free(ws); free(q); free(k); free(v); free(o);
}

sage_problem_t fixed(int B, int H, int Hkv, int N, int d, int causal, int qk, int pv, int layout, int dtype) {
  sage_problem_t p;
  memset(&p, 0, sizeof(p));
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N; p.d = d; p.causal = causal; p.qk_bits = qk; p.pv_bits = pv;
  p.layout = layout; p.dtype = dtype; p.cu_seqlens = nullptr;
  return p;
}
}  // namespace

int main() {
  // fixed-length problems: tails, GQA, both layouts and dtypes, every bit width
  run_case(fixed(1, 2, 2, 256, 64, 0, 8, 8, SAGE_LAYOUT_HND, SAGE_DTYPE_FP16));
  run_case(fixed(2, 4, 2, 300, 128, 1, 4, 16, SAGE_LAYOUT_NHD, SAGE_DTYPE_BF16));
  run_case(fixed(1, 3, 1, 1, 64, 1, 8, 8, SAGE_LAYOUT_HND, SAGE_DTYPE_FP16));
  run_case(fixed(3, 2, 1, 129, 128, 0, 4, 8, SAGE_LAYOUT_HND, SAGE_DTYPE_BF16));
  // varlen batches
  {
    const int cu[] = {0, 5, 9, 300, 301};
    sage_problem_t p = fixed(4, 4, 2, 0, 64, 1, 8, 8, SAGE_LAYOUT_HND, SAGE_DTYPE_FP16);
    p.cu_seqlens = cu;
    run_case(p);
    p.pv_bits = 16; p.dtype = SAGE_DTYPE_BF16; p.causal = 0; p.d = 128;
    run_case(p);
  }
  {
    std::vector<int> cu(70);                          // more than one 64-entry table chunk
    for (int s = 0; s < 70; ++s) cu[s] = s * 37;
    sage_problem_t p = fixed(69, 2, 1, 0, 64, 1, 8, 8, SAGE_LAYOUT_HND, SAGE_DTYPE_FP16);
    p.cu_seqlens = cu.data();
    run_case(p);
  }
  // validation at the edges of the integer ranges: must reject (or accept) without overflow
  size_t n = 0;
  const int big[][8] = {
      {65535, 1, 1, 1 << 23, 128, 1, 8, 8},   {1, 65535, 65535, 1 << 23, 128, 0, 8, 8},
      {2147483647, 1, 1, 1, 64, 0, 8, 8},     {1, 2147483647, 1, 1, 64, 0, 8, 8},
      {1, 1, 1, 2147483647, 64, 0, 8, 8},     {1, 1, 1, -2147483647 - 1, 64, 0, 8, 8},
      {-1, 1, 1, 1, 64, 0, 8, 8},             {65536, 1, 1, 1, 64, 0, 8, 8},
      {300, 200, 100, 1 << 20, 128, 1, 8, 16}, {1, 64, 64, 1 << 23, 64, 0, 8, 8}};
  for (const auto& a : big) {
    sage_problem_t p = fixed(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], SAGE_LAYOUT_HND, SAGE_DTYPE_FP16);
    const int st = sage_attn_workspace_bytes_ex(&p, &n);
    CHECK(st == SAGE_OK || st == SAGE_ERR_INVALID_ARG || st == SAGE_ERR_UNSUPPORTED);
  }
  {
    const int cu[] = {0, 2147483647, -2147483647 - 1};
    sage_problem_t p = fixed(2, 1, 1, 0, 64, 0, 8, 8, SAGE_LAYOUT_HND, SAGE_DTYPE_FP16);
    p.cu_seqlens = cu;
    CHECK(sage_attn_workspace_bytes_ex(&p, &n) != SAGE_OK);
  }
  // the rate probe's argument checks, and a call on a sink of exactly the minimum size
  {
    double ops = 0;
    std::vector<unsigned char> sink(512 * 1024);
    CHECK(sage_mfma_rate_probe(4, 10, sink.data(), sink.size(), &ops, nullptr) == SAGE_ERR_INVALID_ARG);
    CHECK(sage_mfma_rate_probe(0, 0, sink.data(), sink.size(), &ops, nullptr) == SAGE_ERR_INVALID_ARG);
    CHECK(sage_mfma_rate_probe(0, 10, nullptr, sink.size(), &ops, nullptr) == SAGE_ERR_INVALID_ARG);
    CHECK(sage_mfma_rate_probe(0, 10, sink.data(), sink.size() - 1, &ops, nullptr) == SAGE_ERR_WORKSPACE);
    CHECK(sage_mfma_rate_probe(1, 10, sink.data(), sink.size(), &ops, nullptr) == SAGE_OK && ops == 10.0);
  }
  if (g_fail) return 1;
  printf("ok\n");
  return 0;
}
