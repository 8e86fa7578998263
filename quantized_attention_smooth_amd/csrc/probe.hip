// Dense matrix-unit rate probe: the sustained MFMA rate of the chip at the clock it runs at,
// to set the attention kernel's achieved rate beside a measured peak as well as the vendor's.
//
// Every wave runs `iters` rounds of four independent accumulator chains of one matrix
// instruction with register operands: no memory traffic and no other work, two waves per SIMD.
// The launch performs iters * 4 * (ops per instruction) per wave; the caller times it.
#include "sage_internal.h"

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kProbeBlocks = 512;      // two 4-wave workgroups per CU: two waves per SIMD

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe(int iters, float* sink) {
  const int t = threadIdx.x;
  // small nonzero operands that the compiler cannot fold: 0x38 is FP8 E4M3 1.0, 0x08 FP6 E2M3
  // 1.0 in the low six bits, 1 is int8 1; fp16 1.0
  const int pat = KIND == 0 ? 0x01010101 : KIND == 1 ? 0x38383838 : 0x08080808;
  const int x = pat | ((t >> 8) & 0);
  float s = 0.f;
  if (KIND == 0) {
    const v4i a = {x, x, x, x};
    v16i acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) s += (float)acc[c][0];
  } else if (KIND == 1 || KIND == 2) {
    const v8i a = {x, x, x, x, x, x, x, x};
    constexpr int F = KIND == 1 ? 0 : 2;              // format: FP8 E4M3 or FP6 E2M3
    v16f acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[c], F, F, 0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0];
  } else {
    const _Float16 one = (_Float16)(1.0f + (float)((t >> 8) & 0));
    const h8 a = {one, one, one, one, one, one, one, one};
    v16f acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0];
  }
  sink[blockIdx.x * 256 + t] = s;
}

}  // namespace

double mfma_probe_ops(int kind, int iters) {
  const double per = kind == 0 ? 32.0 * 32 * 32 * 2 : kind == 3 ? 32.0 * 32 * 16 * 2 : 32.0 * 32 * 64 * 2;
  return per * 4.0 * iters * 4.0 * kProbeBlocks;       // 4 chains, 4 waves per workgroup
}

size_t mfma_probe_sink_bytes() { return (size_t)kProbeBlocks * 256 * sizeof(float); }

hipError_t launch_mfma_probe(int kind, int iters, float* sink, hipStream_t s) {
  const dim3 grid(kProbeBlocks), blk(256);
  switch (kind) {
    case 0: return launch(mfma_probe<0>, grid, blk, s, iters, sink);
    case 1: return launch(mfma_probe<1>, grid, blk, s, iters, sink);
    case 2: return launch(mfma_probe<2>, grid, blk, s, iters, sink);
    default: return launch(mfma_probe<3>, grid, blk, s, iters, sink);
  }
}

}  // namespace sage
