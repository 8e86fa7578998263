// Internal definitions shared by the gfx950 kernels and the C ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace sage {

// ---- compile-time geometry (exported by sage_get_config) ----
constexpr int BQ = 128;          // queries per workgroup (4 waves x 32) and per Q-mean block
constexpr int BK = 128;          // keys per KV block
constexpr int WAVES = 4;
constexpr int QW = 32;           // queries per wave: one 32-wide MFMA column tile
constexpr float P_RANGE = 448.0f;
constexpr float V_RANGE = 448.0f;
constexpr int VGROUP = 64;       // keys per FP8 MFMA k-step (32x32x64): V^T is stored per 64 keys
constexpr size_t WS_ALIGN = 256;

// ---- problem description ----
// Element strides of the fp16 inputs and output: batch, token, head; channels are contiguous.
// q and o share one set (o has q's shape and layout), k and v the other.
struct Strides {
  long long qb, qt, qh;
  long long kb, kt, kh;
};

// One sequence of the batch.  Fixed-length batches are the uniform case and compute this in
// closed form (Geo::seq); varlen batches read it from a table the library writes into the
// workspace.  Workspace arrays are sequence-major: a sequence's padded rows start at pad0, so
// the per-(sequence, head) sections below are contiguous.
struct Seq {
  int n;           // tokens in the sequence (>= 1)
  int tok0;        // first token in the packed input (varlen), 0 otherwise
  int pad0;        // rows of all earlier sequences, each rounded up to 128
  int unused;
  long long ds0;   // Delta_S elements of all earlier sequences (all heads)
};

struct Dims {
  int B, H, Hkv, N, d, causal, qk_bits, pv_bits;   // B = sequences; N = length (varlen: longest)
  int Npad;   // N rounded up to a multiple of 128 (= BQ = BK)
  int nqb;    // query blocks of the longest sequence
  int nkb;    // KV blocks of the longest sequence
  int varlen; // sequence table in the workspace instead of the uniform closed form
  int bf16;   // inputs and output bf16 (else fp16)
  long long tot_pad;   // sum of the padded lengths
  long long tot_ds;    // Delta_S elements of all sequences and heads
  Strides st;
};

// ---- workspace carve-up (byte offsets, all WS_ALIGN aligned) ----
// Sequence s has Npad_s = its length rounded up to 128 and nb_s = Npad_s / 128 blocks; its
// sections start at row pad0 (block pad0 / 128) of every per-row (per-block) array, heads
// following one another inside it.  A fixed-length batch is [B][heads][Npad] throughout.
//  kcodes : int8  per s: [Hkv][Npad_s][d]       smoothed+quantized K, zero past n (INT4 range:
//                                             packed FP6 E2M3, 24 of every 32 bytes)
//  vcodes : pv_bits 8:  uint8 per s: [Hkv][Npad_s/64][d][64]  FP8 V, transposed per 64-key
//           group; inside a group the byte at position 32*h + b of channel row c holds key
//           32*(b/16) + 8*((b%16)/4) + 4*h + (b%4): the k-slot order of the FP8 MFMA
//           B operand built from the S^T accumulators (see attention kernel)
//           pv_bits 16: fp16 per s: [Hkv][Npad_s/16][d][16]  V itself, transposed per 16-key
//           group; slot 8*((kk/4)%2) + 4*(kk/8) + kk%4 holds key kk of the group: the k-slot
//           order of the fp16 MFMA B operand built from the S^T accumulators
//  qcodes : int8  per s: [H][Npad_s][d]        (INT4 range: packed FP6 E2M3, as kcodes); rows
//           past n hold codes of -mu_Q that no output reads
//  kscale : fp32  per s: [Hkv][nb_s][2]        delta_K per (KV block, lane half)
//  qscale : fp32  per s: [H][Npad_s]           delta_Q per query row
//  muk    : fp32  [B][Hkv][d]
//  ksum   : int64 [B][Hkv][d]                 exact fixed-point K column sums (2^-24 units);
//           bf16 inputs: [B][Hkv][d][12] limbs of 2^(24 i) (units 2^-133)
//  vamax  : u32   [B][Hkv][d]                 bits of max|V| per channel (non-negative floats)
//  vscale : fp32  [B][Hkv][d]                 delta_V
//  muq    : fp32  per s: [H][nb_s][d]
//  muqs   : bf16  per s: [H][nb_s][3][d]       mu_Q split exactly into three bf16 parts
//                                             (x = x1 + x2 + x3), the Delta_S MFMA operand
//  ds     : fp32  per (s, h), from element ds0 of s: the rows of Delta_S * log2(e) / sqrt(d),
//           one per Q block.  Non-causal: nb_s rows of Npad_s keys.  Causal: row qb holds only
//           the keys a causal Q block can see, j < (qb + 1) * 128, packed back to back
//           (ds_row_offset).  Entries past n are -inf, so padded keys drop out of the softmax
//           without a mask.
//  seqs   : Seq [B]                           varlen only: the sequence table
// Delta_S storage: elements per (b, h) and the offset of Q block qb's row inside it.
__host__ __device__ inline size_t ds_head_elems(bool causal, int nqb, int Npad) {
  return causal ? (size_t)BQ * nqb * (nqb + 1) / 2 : (size_t)nqb * Npad;
}
__host__ __device__ inline size_t ds_row_offset(bool causal, int qb, int Npad) {
  return causal ? (size_t)BQ * qb * (qb + 1) / 2 : (size_t)qb * Npad;
}
__host__ __device__ inline int ds_row_len(bool causal, int qb, int Npad) {
  return causal ? (qb + 1) * BQ : Npad;
}

struct Layout {
  size_t kcodes, vcodes, qcodes, kscale, qscale, muk, ksum, vamax, vscale, muq, muqs, ds, seqs, total;
};

inline size_t align_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

inline Layout make_layout(const Dims& D) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  const size_t B = D.B, H = D.H, Hkv = D.Hkv, T = (size_t)D.tot_pad, d = D.d, nb = T / BQ;
  L.kcodes = take(Hkv * T * d);
  L.vcodes = take(Hkv * T * d * (D.pv_bits / 8));
  L.qcodes = take(H * T * d);
  L.kscale = take(Hkv * nb * 2 * 4);
  L.qscale = take(H * T * 4);
  L.muk = take(B * Hkv * d * 4);
  L.ksum = take(B * Hkv * d * 8 * (D.bf16 ? 12 : 1));   // bf16: 12 limbs per exact sum
  L.vamax = take(B * Hkv * d * 4);
  L.vscale = take(B * Hkv * d * 4);
  L.muq = take(H * nb * d * 4);
  L.muqs = take(H * nb * 3 * d * 2);
  L.ds = take((size_t)D.tot_ds * 4);
  L.seqs = take(D.varlen ? B * sizeof(Seq) : 0);
  L.total = off;
  return L;
}

// Device-side view of the batch geometry: per-sequence entries and workspace offsets.
struct Geo {
  const Seq* table;      // null: uniform batch of N-token sequences
  int N, Npad, H, Hkv;
  bool causal;
  long long ds_seq;      // uniform: Delta_S elements per sequence
  Strides st;

  __host__ __device__ Seq seq(int s) const {
    if (table == nullptr) return Seq{N, 0, s * Npad, 0, (long long)s * ds_seq};
    return table[s];
  }
};

__host__ __device__ inline int seq_blocks(const Seq& q) { return (q.n + BQ - 1) / BQ; }
// row offsets of head h's padded rows (codes, per-row scales) and block offsets (per-block data)
__host__ __device__ inline size_t rows_off(const Seq& q, int heads, int h) {
  return (size_t)q.pad0 * heads + (size_t)h * seq_blocks(q) * BQ;
}
__host__ __device__ inline size_t blocks_off(const Seq& q, int heads, int h) {
  return (size_t)(q.pad0 / BQ) * heads + (size_t)h * seq_blocks(q);
}
__host__ __device__ inline size_t ds_off(const Seq& q, bool causal, int h) {
  const int nb = seq_blocks(q);
  return (size_t)q.ds0 + (size_t)h * ds_head_elems(causal, nb, nb * BQ);
}

inline Geo make_geo(const Dims& D, const void* seq_table) {
  Geo g;
  g.table = D.varlen ? static_cast<const Seq*>(seq_table) : nullptr;
  g.N = D.N; g.Npad = D.Npad; g.H = D.H; g.Hkv = D.Hkv;
  g.causal = D.causal != 0;
  g.ds_seq = (long long)D.H * (long long)ds_head_elems(D.causal != 0, D.nqb, D.Npad);
  g.st = D.st;
  return g;
}

struct Ptrs {
  const __half* q;
  const __half* k;
  const __half* v;
  __half* o;
  int8_t* kcodes;
  uint8_t* vcodes;
  int8_t* qcodes;
  float* kscale;
  float* qscale;
  float* muk;
  unsigned long long* ksum;
  unsigned int* vamax;
  float* vscale;
  float* muq;
  uint16_t* muqs;
  float* ds;
  Seq* seqs;
};

inline Ptrs carve(void* ws, const Layout& L, const void* q, const void* k, const void* v, void* o) {
  char* w = static_cast<char*>(ws);
  Ptrs p;
  p.q = static_cast<const __half*>(q);
  p.k = static_cast<const __half*>(k);
  p.v = static_cast<const __half*>(v);
  p.o = static_cast<__half*>(o);
  p.kcodes = reinterpret_cast<int8_t*>(w + L.kcodes);
  p.vcodes = reinterpret_cast<uint8_t*>(w + L.vcodes);
  p.qcodes = reinterpret_cast<int8_t*>(w + L.qcodes);
  p.kscale = reinterpret_cast<float*>(w + L.kscale);
  p.qscale = reinterpret_cast<float*>(w + L.qscale);
  p.muk = reinterpret_cast<float*>(w + L.muk);
  p.ksum = reinterpret_cast<unsigned long long*>(w + L.ksum);
  p.vamax = reinterpret_cast<unsigned int*>(w + L.vamax);
  p.vscale = reinterpret_cast<float*>(w + L.vscale);
  p.muq = reinterpret_cast<float*>(w + L.muq);
  p.muqs = reinterpret_cast<uint16_t*>(w + L.muqs);
  p.ds = reinterpret_cast<float*>(w + L.ds);
  p.seqs = reinterpret_cast<Seq*>(w + L.seqs);
  return p;
}

// Workgroup ids are dealt to the 8 XCDs (each with its own L2) round-robin: id i runs on XCD
// i % 8.  xcd_remap(i, total) renumbers them so that XCD x works through one contiguous share
// of [0, total), shares differing in size by at most one.
__device__ inline int xcd_remap(int bid, int total) {
  const int q = total / 8, r = total % 8;
  const int x = bid % 8, k = bid / 8;
  return x * q + min(x, r) + k;
}
// A raw buffer resource over [base, base + bytes): loads past the end return zero and stores
// past it are dropped.  Buffer builtins exist only for the GPU target, so every use sits in
// device-pass code (#if defined(__HIP_DEVICE_COMPILE__)).
#if defined(__HIP_DEVICE_COMPILE__)
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
#endif
// Launch kernel k on stream s and return the status of this launch itself.  (A launch written as
// k<<<...>>>(...) followed by hipGetLastError() would also report an error left on the thread by
// an unrelated earlier call.)  The arguments are converted to the kernel's parameter types.
template <typename... P, typename... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A) && sizeof...(P) > 0, "kernel argument count");
  std::tuple<P...> vals(static_cast<P>(std::forward<A>(args))...);
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, s);
      },
      vals);
}

// ---- launchers (return the hipError_t of the launch) ----
// varlen: copy the host-built sequence table into the workspace (kernel arguments, no host
// buffer outlives the call)
hipError_t launch_seq_table(const Seq* host, int n, Seq* dev, hipStream_t s);
hipError_t launch_prologue(const Dims& D, const Ptrs& P, hipStream_t s);
hipError_t launch_attention(const Dims& D, const Ptrs& P, hipStream_t s);
hipError_t launch_qk_tile(const Dims& D, const Ptrs& P, int b, int h, int qb, int kb, int32_t* out,
                          hipStream_t s);
// matrix-unit rate probe: ops per launch, sink size, launch (kind 0 INT8, 1 FP8, 2 FP6, 3 fp16)
double mfma_probe_ops(int kind, int iters);
size_t mfma_probe_sink_bytes();
hipError_t launch_mfma_probe(int kind, int iters, float* sink, hipStream_t s);
hipError_t launch_debug_copy(const Dims& D, const Ptrs& P, hipStream_t s, float* mu_k, int8_t* k_codes,
                             float* k_scales, uint8_t* v_codes, float* v_scales, float* mu_q,
                             int8_t* q_codes, float* q_scales, float* delta_s);

}  // namespace sage
