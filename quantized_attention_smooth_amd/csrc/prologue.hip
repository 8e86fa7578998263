// Quantize/smooth prologue for the SageAttention2 forward on gfx950.
//
// Page "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and Per-thread
// INT4 Quantization" (mlsanity.com, arXiv 2411.10958), section "Abstract (arXiv)": K and Q are
// smoothed and quantized to 4-bit (here also 8-bit) integers at thread granularity, V to FP8.
// pith.science verdict on arXiv 2505.21136, key "key_machinery": per-channel V scale
// max|V| / V_r.
//
// The codec kernels stream HBM: each reads its fp16 input once (K and V twice: statistics, then
// quantization) and writes 1-byte codes plus a few scales.  Delta_S (the Q-smoothing bias,
// mu_Q . gamma_K per Q block and key) reads K a third time and writes 4 bytes per (Q block, key).
//
// Bit-exactness: the channel means are exact sums.  Every fp16 value is an integer multiple of
// 2^-24 below 2^16, so a sum of up to 256 of them is exact in fp64 (below 2^24, 48 bits of
// 2^-24 units); whole-sequence K sums cross workgroups as int64 counts of 2^-24 units.  Each
// mean is one fp64 division rounded to fp32.  Smoothing is one fp32 subtraction; codes are
// round-half-even of one fp32 product with the correctly rounded fp32 reciprocal R / amax;
// scales are the correctly rounded fp32 quotient amax / R.  None of these depend on the
// order of the parallel reduction, so codes and scales are reproducible bit for bit.
#include <type_traits>

#include "sage_internal.h"

namespace sage {

namespace {

// 8 consecutive input elements (fp16 or bf16) as raw bits, converted on use
template <typename T> __device__ inline float bits_to_float(uint16_t b);
template <> __device__ inline float bits_to_float<__half>(uint16_t b) { return __half2float(__ushort_as_half(b)); }
template <> __device__ inline float bits_to_float<__bf16>(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T>
struct In8 {
  uint16_t b[8];
  __device__ float f(int e) const { return bits_to_float<T>(b[e]); }
};

template <typename T>
__device__ inline In8<T> load8(const T* p) {
  In8<T> r;
  *reinterpret_cast<uint4*>(r.b) = *reinterpret_cast<const uint4*>(p);
  return r;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// INT4-range codes (|code| <= 7) go to the attention kernel as OCP FP6 E2M3 numbers, which hold
// the integers -7..7 exactly and feed the FP6 MFMA at twice the FP8/INT8 rate.  Each 32-channel
// group of a row occupies a 32-byte slot: 24 bytes of packed 6-bit codes (channel i of the group
// at bits 6i..6i+5) and 8 zero bytes, so rows keep d bytes and the FP8/INT8 tile geometry.
__device__ inline uint32_t e2m3_bits(float x) {        // x integer in [-7, 7]
  // magnitudes 0..7 are E2M3 0x00 0x08 0x10 0x14 0x18 0x1A 0x1C 0x1E: one byte each of a
  // 64-bit constant, picked by a shift (no branches)
  const int a = (int)fabsf(x);
  const uint32_t mag = (uint32_t)(0x1E1C1A1814100800ull >> (8 * a)) & 0xFFu;
  return mag | (x < 0.f ? 0x20u : 0u);
}

// Store the 8 codes of channels 8 cq .. 8 cq + 7 of one row (row points at its d code bytes).
// FP6: the four threads of a 32-channel slot are consecutive lanes (cq & 3 = 0..3); they swap
// their 48-bit packs so that each writes one aligned 8-byte word of the slot.
template <bool FP6>
__device__ inline void store_codes(int8_t* row, int cq, const float (&x)[8]) {
  if (!FP6) {
    union { int8_t c[8]; uint2 u; } out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out.c[e] = (int8_t)(int)x[e];
    *reinterpret_cast<uint2*>(row + cq * 8) = out.u;
    return;
  }
  unsigned long long mine = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) mine |= (unsigned long long)e2m3_bits(x[e]) << (6 * e);
  const int j = cq & 3;
  // slot bits [48 t, 48 t + 48) hold thread t's pack; word j covers bits [64 j, 64 j + 64)
  const unsigned long long nxt = __shfl_down(mine, 1, 4);   // pack of thread j + 1 (same slot)
  // j = 0, 1, 2: bits [16 j, 64) of this pack and the first 16 (j + 1) bits of the next one;
  // j = 3: bytes 24..31 of the slot, padding
  const unsigned long long word = j < 3 ? (mine >> (16 * j)) | (nxt << (48 - 16 * j)) : 0ull;
  *reinterpret_cast<uint2*>(row + 32 * (cq >> 2) + 8 * j) = make_uint2((uint32_t)word, (uint32_t)(word >> 32));
}

// ---------------------------------------------------------------------------------------
// Exact sums of bf16 values.  A bf16 number is an integer m < 2^8 times 2^p in units of 2^-133
// (p = biased exponent - 1 for normal numbers, 0 for subnormals), so a column sum of up to
// 2^23 of them is an integer below 2^284.  It is kept as kLimbs signed int64 limbs of weight
// 2^(24 i): each value adds m * 2^(p mod 24) < 2^32 to limb p div 24, so no limb can overflow
// (2^23 terms * 2^32 < 2^63) whatever the order of the additions.  superacc_value turns the
// limbs into the correctly rounded fp64 value of the sum (round to nearest even), which is
// what the mean needs: mu = RN32(RN64(sum) / n), the same rule as for fp16 inputs.
// ---------------------------------------------------------------------------------------
constexpr int kLimbs = 12;

__device__ inline void superacc_add(unsigned long long* acc, uint16_t bits) {
  const int e = (bits >> 7) & 0xFF;
  const int m = e ? (bits & 0x7F) | 0x80 : bits & 0x7F;
  const int p = e ? e - 1 : 0;
  const long long c = (long long)m << (p % 24);
  atomicAdd(acc + p / 24, (unsigned long long)((bits & 0x8000) ? -c : c));
}

__device__ inline double superacc_value(const unsigned long long* limbs) {
  long long M[kLimbs];
  long long carry = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {            // normalise: every limb in [0, 2^24)
    const long long x = (long long)limbs[i] + carry;
    carry = x >> 24;                            // arithmetic shift: floor division
    M[i] = x - (carry << 24);
  }
  const bool neg = carry < 0;                   // the total is -2^288 + sum M_i 2^(24 i)
  if (neg) {                                    // magnitude: 2^288 - sum M_i 2^(24 i)
    long long c1 = 1;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) {
      const long long x = ((1LL << 24) - 1 - M[i]) + c1;
      c1 = x >> 24;
      M[i] = x & ((1LL << 24) - 1);
    }
  }
  int t = -1;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i)
    if (M[i] != 0) t = i;
  if (t < 0) return 0.0;
  // 96-bit window of the top four limbs, the rest as a sticky bit
  unsigned __int128 W = 0;
  bool sticky = false;
#pragma unroll
  for (int i = kLimbs - 1; i >= 0; --i) {
    if (i <= t && i >= t - 3) W = (W << 24) | (unsigned __int128)M[i];
    else if (i < t - 3 && M[i] != 0) sticky = true;
  }
  for (int i = t - 3; i < 0; ++i) W <<= 24;     // windows that start below limb 0
  const unsigned long long hi = (unsigned long long)(W >> 64), lo = (unsigned long long)W;
  const int bitlen = hi ? 128 - __clzll(hi) : 64 - __clzll(lo);
  int shift = bitlen - 53;                      // >= 20: the top limb is nonzero
  unsigned long long mant = (unsigned long long)(W >> shift);
  const unsigned __int128 rem = W & (((unsigned __int128)1 << shift) - 1);
  const unsigned __int128 half = (unsigned __int128)1 << (shift - 1);
  if (rem > half || (rem == half && (sticky || (mant & 1)))) {
    if (++mant >> 53) { mant >>= 1; ++shift; }
  }
  const double r = ldexp((double)mant, shift + 24 * (t - 3) - 133);
  return neg ? -r : r;
}

// ---------------------------------------------------------------------------------------
// zero the atomically reduced statistics
// ---------------------------------------------------------------------------------------
__global__ void init_stats(unsigned long long* ksum, unsigned int* vamax, int n, int limbs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    for (int l = 0; l < limbs; ++l) ksum[(size_t)i * limbs + l] = 0ull;
    vamax[i] = 0u;
  }
}

// ---------------------------------------------------------------------------------------
// K channel sums and V channel abs-max, per (sequence, kv head).  The sums are exact: fp16
// inputs in fp64 within a workgroup and int64 fixed point across; bf16 inputs in the limb
// accumulator above (LDS within a workgroup, int64 atomics across).  VSTATS = false (V kept in
// 16-bit floats) skips V entirely.
// Workgroup (bx, by) of a (ceil(longest / 256), B*Hkv) tiling, 256 threads; thread = (row slot,
// 8-channel chunk).  Runs inside stats_and_q.
// ---------------------------------------------------------------------------------------
template <int D, typename T>
struct KvStatsSmem {
  static constexpr int RPP = 256 / (D / 8);
  static constexpr bool BF = std::is_same<T, __bf16>::value;
  double ls[BF ? 1 : RPP][D];
  float lm[RPP][D];
  unsigned long long acc[BF ? D * kLimbs : 1];
};

// (bx, by): the workgroup's token tile and (sequence, kv head)
template <int D, bool VSTATS, typename T>
__device__ inline void kv_stats_body(const T* __restrict__ k, const T* __restrict__ v,
                                     unsigned long long* __restrict__ ksum, unsigned int* __restrict__ vamax,
                                     const Geo& g, int bx, int by, KvStatsSmem<D, T>& sm) {
  constexpr int TPR = D / 8;      // threads per row
  constexpr int RPP = 256 / TPR;  // rows per pass
  constexpr int TOK = 256;        // tokens per workgroup
  constexpr bool BF = std::is_same<T, __bf16>::value;
  auto& ls = sm.ls;
  auto& lm = sm.lm;
  auto& acc = sm.acc;
  const int tid = threadIdx.x, cq = tid % TPR, r0 = tid / TPR;
  const size_t bh = by;                         // (sequence, kv head)
  const int sidx = (int)bh / g.Hkv, hk = (int)bh % g.Hkv;
  const Seq sq = g.seq(sidx);
  const int N = sq.n;
  if (bx * TOK >= N) return;
  const long long base = sidx * g.st.kb + (long long)sq.tok0 * g.st.kt + hk * g.st.kh;
  const T* kb = k + base;
  const T* vb = v + base;
  // Sums of at most TOK fp16 values are exact in fp64: every term is a multiple of 2^-24 and the
  // total stays below 2^24 < 2^(53 - 24).  The workgroup's exact total is then handed to the
  // cross-workgroup reduction as an int64 count of 2^-24 units.
  double s[8];
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { s[e] = 0.0; mx[e] = 0.f; }
  if (BF) {
    for (int i = tid; i < D * kLimbs; i += 256) acc[i] = 0ull;
    __syncthreads();
  }
  const int tok0 = bx * TOK;
  // 4 passes at a time, loads issued before use: rows past N read row N - 1 (in bounds) and are
  // skipped afterwards, so no load waits behind its own branch
  constexpr int CH = 4;
  for (int p0 = 0; p0 < TOK / RPP; p0 += CH) {
    In8<T> kr[CH], vr[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const long long off = (long long)min(tok0 + (p0 + i) * RPP + r0, N - 1) * g.st.kt + cq * 8;
      kr[i] = load8(kb + off);
      if (VSTATS) vr[i] = load8(vb + off);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (tok0 + (p0 + i) * RPP + r0 >= N) continue;
      if (BF) {
#pragma unroll
        for (int e = 0; e < 8; ++e) superacc_add(&acc[(cq * 8 + e) * kLimbs], kr[i].b[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += (double)kr[i].f(e);
      }
      if (VSTATS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf(vr[i].f(e)));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (!BF) ls[r0][cq * 8 + e] = s[e];
    lm[r0][cq * 8 + e] = mx[e];
  }
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    double t = 0.0;
    float m = 0.f;
    for (int r = 0; r < RPP; ++r) {
      if (!BF) t += ls[r][c];
      m = fmaxf(m, lm[r][c]);
    }
    if (!BF) atomicAdd(&ksum[bh * D + c], (unsigned long long)(long long)(t * 16777216.0));   // exact integer
    if (VSTATS) atomicMax(&vamax[bh * D + c], __float_as_uint(m));   // order of non-negative floats
  }
  if (BF) {
    for (int i = tid; i < D * kLimbs; i += 256)
      if (acc[i] != 0ull) atomicAdd(&ksum[bh * D * kLimbs + i], acc[i]);
  }
}

// ---------------------------------------------------------------------------------------
// fp16 V for the fp16 P V MFMA: the 128 keys of KV block kb, transposed into 8 groups of 16
// keys, [group][channel][16 slots]; key kk of a group sits in slot 8 ((kk / 4) % 2) +
// 4 (kk / 8) + kk % 4, the k-slot order of the fp16 MFMA B operand the attention kernel
// builds from its S^T accumulators.  A thread takes 4 consecutive keys (4 consecutive slots:
// one 8-byte LDS write per channel).  LDS rows (32 bytes) are XOR-permuted within each run of
// 8 (row ^ (row / 8) % 8) so that the 8 channels 8 apart a wave writes at once fall on
// distinct banks; the copy-out undoes it.
// ---------------------------------------------------------------------------------------
__device__ inline int v16_lds_row(int row) { return row ^ ((row >> 3) & 7); }

template <int D, typename T>
__device__ inline void store_v16(const T* __restrict__ vbase, long long tstride, uint8_t* vt,
                                 uint8_t* __restrict__ dst, int kb, int N, int tid, int cq, int r0) {
  constexpr int TPR = D / 8, RPP = 256 / TPR, G4 = BK / 4 / RPP;
#pragma unroll
  for (int p = 0; p < G4; ++p) {
    const int jl0 = 4 * (p * RPP + r0);        // first of the thread's 4 keys within the block
    const int g = jl0 >> 4, kk = jl0 & 15;
    const int quad = 2 * ((kk >> 2) & 1) + (kk >> 3);   // slots 4 quad .. 4 quad + 3
    uint16_t x[4][8];
    In8<T> vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = load8(vbase + min(kb * BK + jl0 + i, N - 1) * tstride + cq * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = kb * BK + jl0 + i < N;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = valid ? vr[i].b[e] : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = g * D + cq * 8 + e;
      const uint2 w2 = make_uint2((uint32_t)x[0][e] | ((uint32_t)x[1][e] << 16),
                                  (uint32_t)x[2][e] | ((uint32_t)x[3][e] << 16));
      *reinterpret_cast<uint2*>(vt + v16_lds_row(row) * 32 + quad * 8) = w2;
    }
  }
  __syncthreads();
  for (int ch = tid; ch < BK * D * 2 / 16; ch += 256) {
    const int row = ch >> 1;
    *reinterpret_cast<uint4*>(dst + ch * 16) =
        *reinterpret_cast<const uint4*>(vt + v16_lds_row(row) * 32 + (ch & 1) * 16);
  }
}

// ---------------------------------------------------------------------------------------
// K smoothing + quantization and V FP8 quantization for one KV block of 128 keys.
// grid (blocks of the longest sequence, B*Hkv), 256 threads.
// K group: keys 8a + 4h + r of the block share the scale of lane half h (one scale per
// lane of the 32x32 integer MFMA accumulator that holds those keys).
// V codes are written transposed per 64-key group in the FP8 MFMA k-slot order; with PV16
// V itself (fp16) is written transposed per 16-key group in the fp16 MFMA k-slot order.
// ---------------------------------------------------------------------------------------
template <int D, bool PV16, typename T, bool QK4>
__global__ __launch_bounds__(256) void kv_quant(const T* __restrict__ k, const T* __restrict__ v,
                                                const unsigned long long* __restrict__ ksum,
                                                const unsigned int* __restrict__ vamax,
                                                int8_t* __restrict__ kcodes, uint8_t* __restrict__ vcodes,
                                                float* __restrict__ kscale, float* __restrict__ muk_out,
                                                float* __restrict__ vscale, Geo g, float R) {
  constexpr int TPR = D / 8, RPP = 256 / TPR, PASSES = BK / RPP;
  static_assert(RPP % 8 == 0, "a thread's rows must share (row % 8)");
  __shared__ float red[WAVES][2];
  __shared__ __attribute__((aligned(16))) uint8_t vt[BK * D * (PV16 ? 2 : 1)];
  const int tid = threadIdx.x, cq = tid % TPR, r0 = tid / TPR, lane = tid % 64, w = tid / 64;
  const int kb = blockIdx.x;
  const size_t bh = blockIdx.y;                 // (sequence, kv head)
  const int sidx = (int)bh / g.Hkv, hk = (int)bh % g.Hkv;
  const Seq sq = g.seq(sidx);
  if (kb >= seq_blocks(sq)) return;
  const int N = sq.n;
  const long long ts = g.st.kt;
  const T* kbase = k + sidx * g.st.kb + (long long)sq.tok0 * ts + hk * g.st.kh;
  const T* vbase = v + sidx * g.st.kb + (long long)sq.tok0 * ts + hk * g.st.kh;
  const size_t rows = rows_off(sq, g.Hkv, hk);  // this head's padded rows in the code arrays

  float mu[8], vinv[8];
  // this thread's 8 channel sums and abs-maxima, loaded together (fp16: 64 + 32 contiguous bytes)
  unsigned long long ks8[8];
  uint32_t va8[8];
  if (!std::is_same<T, __bf16>::value) {
    const uint4* kp = reinterpret_cast<const uint4*>(ksum + bh * D + cq * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = kp[i];
      ks8[2 * i] = ((unsigned long long)w.y << 32) | w.x;
      ks8[2 * i + 1] = ((unsigned long long)w.w << 32) | w.z;
    }
  }
  if (!PV16) {
    const uint4* vp = reinterpret_cast<const uint4*>(vamax + bh * D + cq * 8);
    const uint4 w0 = vp[0], w1 = vp[1];
    va8[0] = w0.x; va8[1] = w0.y; va8[2] = w0.z; va8[3] = w0.w;
    va8[4] = w1.x; va8[5] = w1.y; va8[6] = w1.z; va8[7] = w1.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = cq * 8 + e;
    if (std::is_same<T, __bf16>::value) {
      mu[e] = (float)(superacc_value(&ksum[(bh * D + c) * kLimbs]) / (double)N);
    } else {
      const long long S = (long long)ks8[e];
      mu[e] = (float)((double)S / ((double)N * 16777216.0));
    }
    const float va = PV16 ? 0.f : __uint_as_float(va8[e]);
    vinv[e] = va > 0.f ? V_RANGE / va : 0.f;
    if (kb == 0 && r0 == 0) {
      muk_out[bh * D + c] = mu[e];
      if (!PV16) vscale[bh * D + c] = va / V_RANGE;
    }
  }

  // gamma_K = RN32(K - mu_K); every row of this thread has the same (row % 8)
  // loads issued before use (rows past N read row N - 1 and are zeroed afterwards)
  float gk[PASSES][8];
  float am = 0.f;
  In8<T> kr[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) kr[p] = load8(kbase + min(kb * BK + p * RPP + r0, N - 1) * ts + cq * 8);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const bool valid = kb * BK + p * RPP + r0 < N;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gk[p][e] = valid ? kr[p].f(e) - mu[e] : 0.f;
      am = fmaxf(am, fabsf(gk[p][e]));
    }
  }
  const int hgrp = (r0 & 7) >> 2;
  float a0 = wave_max(hgrp == 0 ? am : 0.f);
  float a1 = wave_max(hgrp == 1 ? am : 0.f);
  if (lane == 0) { red[w][0] = a0; red[w][1] = a1; }
  __syncthreads();
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) amax = fmaxf(amax, red[i][hgrp]);
  const float inv = amax > 0.f ? R / amax : 0.f;
  if (tid < 2) {
    float a = 0.f;
    for (int i = 0; i < WAVES; ++i) a = fmaxf(a, red[i][tid]);
    kscale[(blocks_off(sq, g.Hkv, hk) + kb) * 2 + tid] = a / R;
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = kb * BK + p * RPP + r0;   // < Npad: rows past N get zero codes
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = fminf(fmaxf(rintf(gk[p][e] * inv), -R), R);
    store_codes<QK4>(kcodes + (rows + row) * D, cq, x);
  }

  if (PV16) {
    store_v16<D>(vbase, ts, vt, vcodes + (rows + (size_t)kb * BK) * D * 2, kb, N, tid, cq, r0);
    return;
  }

  // V: per-channel FP8, transposed into [group u][channel][slot] in LDS, then streamed out.
  // A thread takes 4 consecutive keys: their codes fill 4 consecutive slots, one 32-bit LDS
  // write per channel.  The 16-byte chunk of a channel row is XOR-swizzled by channel bits 3-4
  // against bank conflicts (lanes of a wave differ in channel by multiples of 8) and unswizzled
  // on the way out.
  constexpr int G4 = BK / 4 / RPP;             // passes of 4-key groups
#pragma unroll
  for (int p = 0; p < G4; ++p) {
    const int jl0 = 4 * (p * RPP + r0);        // first of the thread's 4 keys within the block
    const int u = jl0 >> 6, jj = jl0 & 63;
    const int base = 32 * ((jj >> 2) & 1) + 16 * (jj >> 5) + 4 * ((jj >> 3) & 3);   // slot of key jj
    float x[4][8];
    In8<T> vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = load8(vbase + min(kb * BK + jl0 + i, N - 1) * ts + cq * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = kb * BK + jl0 + i < N;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = valid ? fminf(fmaxf(vr[i].f(e) * vinv[e], -V_RANGE), V_RANGE) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = cq * 8 + e;
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0][e], x[1][e], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(x[2][e], x[3][e], word, true);
      const int phys = (((base >> 4) ^ ((c >> 3) & 3)) << 4) | (base & 15);
      *reinterpret_cast<int*>(&vt[(u * D + c) * VGROUP + phys]) = word;
    }
  }
  __syncthreads();
  uint8_t* dst = vcodes + (rows + (size_t)kb * BK) * D;
  for (int ch = tid; ch < 2 * D * VGROUP / 16; ch += 256) {
    const int rowc = ch >> 2, c = rowc % D;    // row = group * D + channel
    const int src = rowc * VGROUP + (((ch & 3) ^ ((c >> 3) & 3)) << 4);
    *reinterpret_cast<uint4*>(dst + ch * 16) = *reinterpret_cast<const uint4*>(vt + src);
  }
}

// ---------------------------------------------------------------------------------------
// Q smoothing (per 128-row block mean) + per-row quantization.
// Workgroup (bx, by) of a (blocks of the longest sequence, B*H) tiling, 256 threads.  Runs
// inside stats_and_q.
// ---------------------------------------------------------------------------------------
template <int D, typename T>
struct QQuantSmem {
  static constexpr int RPP = 256 / (D / 8);
  static constexpr bool BF = std::is_same<T, __bf16>::value;
  double ls[BF ? 1 : RPP][D];
  float lmu[D];
  unsigned long long acc[BF ? D * kLimbs : 1];
};

// (bx, by): the workgroup's Q block and (sequence, head)
template <int D, typename T, bool QK4>
__device__ inline void q_quant_body(const T* __restrict__ q, int8_t* __restrict__ qcodes,
                                    float* __restrict__ qscale, float* __restrict__ muq,
                                    uint16_t* __restrict__ muqs, const Geo& g, float R, int bx, int by,
                                    QQuantSmem<D, T>& sm) {
  constexpr int TPR = D / 8, RPP = 256 / TPR, PASSES = BQ / RPP;
  constexpr bool BF = std::is_same<T, __bf16>::value;
  auto& ls = sm.ls;
  auto& lmu = sm.lmu;
  auto& acc = sm.acc;
  const int tid = threadIdx.x, cq = tid % TPR, r0 = tid / TPR;
  const int qb = bx;
  const int sidx = by / g.H, h = by % g.H;
  const Seq sq = g.seq(sidx);
  if (qb >= seq_blocks(sq)) return;
  const int N = sq.n;
  const long long ts = g.st.qt;
  const T* qbase = q + sidx * g.st.qb + (long long)sq.tok0 * ts + h * g.st.qh;
  const size_t rows = rows_off(sq, g.H, h), blk = blocks_off(sq, g.H, h) + qb;
  const int nvalid = min(BQ, N - qb * BQ);

  // block sums are exact: fp16 in fp64 (at most 128 terms, multiples of 2^-24, below 2^24),
  // bf16 in the limb accumulator
  float x[PASSES][8];
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
  if (BF) {
    for (int i = tid; i < D * kLimbs; i += 256) acc[i] = 0ull;
    __syncthreads();
  }
  // every load is issued before any is used: rows past N read row N - 1 (in bounds) and are
  // zeroed afterwards, so no load sits behind a branch that would wait for it on its own
  In8<T> raw[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
    raw[p] = load8(qbase + min(qb * BQ + p * RPP + r0, N - 1) * ts + cq * 8);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const bool valid = qb * BQ + p * RPP + r0 < N;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[p][e] = valid ? raw[p].f(e) : 0.f;
      if (!BF) s[e] += (double)x[p][e];
    }
    if (BF && valid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) superacc_add(&acc[(cq * 8 + e) * kLimbs], raw[p].b[e]);
    }
  }
  if (!BF) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ls[r0][cq * 8 + e] = s[e];
  }
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    double t = 0.0;
    if (BF) {
      t = superacc_value(&acc[c * kLimbs]);
    } else {
      for (int r = 0; r < RPP; ++r) t += ls[r][c];
    }
    const float m = (float)(t / (double)nvalid);
    lmu[c] = m;
    muq[blk * D + c] = m;
    // exact three-part bf16 split of the mean, the A operand of the Delta_S GEMM
    const __bf16 b1 = (__bf16)m;
    const float r1 = m - (float)b1;
    const __bf16 b2 = (__bf16)r1;
    const __bf16 b3 = (__bf16)(r1 - (float)b2);
    uint16_t* dst = muqs + blk * 3 * D + c;
    dst[0] = __builtin_bit_cast(uint16_t, b1);
    dst[D] = __builtin_bit_cast(uint16_t, b2);
    dst[2 * D] = __builtin_bit_cast(uint16_t, b3);
  }
  __syncthreads();
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = lmu[cq * 8 + e];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = qb * BQ + p * RPP + r0;
    const bool valid = row < N;
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[p][e] = valid ? x[p][e] - mu[e] : 0.f;   // gamma_Q = RN32(Q - mu_Q)
      am = fmaxf(am, fabsf(x[p][e]));
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
    const float inv = am > 0.f ? R / am : 0.f;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(rintf(x[p][e] * inv), -R), R);
    store_codes<QK4>(qcodes + (rows + row) * D, cq, y);
    if (cq == 0) qscale[rows + row] = am / R;
  }
}

// ---------------------------------------------------------------------------------------
// K/V channel statistics and the Q prologue in one launch (they are independent): workgroups
// 0 .. nks - 1 take the statistics tiles, the rest the Q blocks, so the Q blocks' load and
// reduction latency overlaps the statistics stream and one launch (and its tail) is saved.
// grid (nks + nqb * B*H), 256 threads.
// ---------------------------------------------------------------------------------------
template <int D, bool VSTATS, typename T, bool QK4>
__global__ __launch_bounds__(256) void stats_and_q(const T* __restrict__ k, const T* __restrict__ v,
                                                   unsigned long long* __restrict__ ksum,
                                                   unsigned int* __restrict__ vamax, const T* __restrict__ q,
                                                   int8_t* __restrict__ qcodes, float* __restrict__ qscale,
                                                   float* __restrict__ muq, uint16_t* __restrict__ muqs, Geo g,
                                                   float R, int stx, int nks, int nqb) {
  __shared__ union U {
    KvStatsSmem<D, T> ks;
    QQuantSmem<D, T> qq;
  } sm;
  const int i = blockIdx.x;
  if (i < nks) kv_stats_body<D, VSTATS, T>(k, v, ksum, vamax, g, i % stx, i / stx, sm.ks);
  else q_quant_body<D, T, QK4>(q, qcodes, qscale, muq, muqs, g, R, (i - nks) % nqb, (i - nks) / nqb, sm.qq);
}

// ---------------------------------------------------------------------------------------
// Delta_S[qb, j] = sum_c mu_Q[qb, c] * gamma_K[j, c], stored times log2(e)/sqrt(d).
//
// A GEMM (Q blocks x keys x channels) on the bf16 MFMA at fp32-class accuracy: both fp32
// factors are split exactly into three bf16 parts, x = x1 + x2 + x3 (8 significant bits each,
// 24 in all), and the six cross products whose weight is at least 2^-16 of the leading one
// are accumulated, smallest first (x3y1 + x2y2 + x1y3 + x2y1 + x1y2 + x1y1); the dropped
// terms are below 2^-24 of it.  The bf16 MFMA accumulates in fp32 (unlike the FP8 one).
//
// One workgroup per (32 NU Q blocks of one query head, 256 keys), 256 threads, NU = 1 or 2.
// The Q blocks' mu_Q parts (split by the Q prologue) are copied to LDS once and read there by
// all four waves; wave w owns keys 64 w .. 64 w + 63 of the tile, loads their rows up front
// (one memory round trip), forms gamma_K = RN32(K - mu_K) and its split one 16-channel k-step
// at a time, and accumulates NU x 2 MFMA tiles of 32 Q blocks x 32 keys.  Workgroup ids run over
// (Q-block tile, query head of the group, key tile, sequence, kv head), fastest first, split into
// one contiguous share per XCD (own L2): the workgroups that read one key tile are adjacent
// and on one XCD, so the keys come from HBM about once however many Q blocks and query heads
// use them, and each XCD's share holds whole kv heads of every sequence (even varlen shares).
// Causal: Q block qb stores keys j < (qb + 1) * 128; workgroups and waves whose keys no row of
// theirs stores exit early, and a 32-row tile with no such row is multiplied but not stored.
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int DS_KT = 256;    // keys per workgroup: 64 per wave, two 32-column MFMA tiles

// QT Q blocks per workgroup (NU = QT / 32 MFMA row tiles)
template <int D, int QT>
struct DsSmem {
  // one Q block's three bf16 parts of D channels, plus 16 bytes: the 32 lanes of an operand
  // read (32 consecutive Q blocks, one 16-byte chunk each) then fall on distinct banks
  static constexpr int ROW = 3 * D * 2 + 16;
  __attribute__((aligned(16))) uint8_t a[QT * ROW];
  __attribute__((aligned(16))) float muk[D];
};

struct Split3 {
  bf16x8 p[3];
};

// x = x1 + x2 + x3 exactly, in pairs: the packed fp32 -> bf16 convert rounds two elements to
// nearest even at once, and a bf16 pair widens back to fp32 by a shift (low) and a mask (high).
// Each residual x - x1 and x - x1 - x2 is exact in fp32 (the rounding error of a narrower format).
__device__ inline uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline Split3 split3(const float (&x)[8]) {
  uint32_t w[3][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[2 * i], b = x[2 * i + 1];
    const uint32_t w1 = bf16_pair(a, b);
    const float ra = a - bf16_lo(w1), rb = b - bf16_hi(w1);
    const uint32_t w2 = bf16_pair(ra, rb);
    w[0][i] = w1;
    w[1][i] = w2;
    w[2][i] = bf16_pair(ra - bf16_lo(w2), rb - bf16_hi(w2));   // at most 8 significant bits remain: exact
  }
  Split3 s;
#pragma unroll
  for (int p = 0; p < 3; ++p) s.p[p] = __builtin_bit_cast(bf16x8, (uint4){w[p][0], w[p][1], w[p][2], w[p][3]});
  return s;
}

// Store v at byte offset off of [base, base + bytes) through a buffer resource: a store at or past
// the end is dropped by the hardware's range check, so masked elements cost no branch.
__device__ inline void store_or_drop(float* base, uint32_t bytes, uint32_t off, float v) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), make_rsrc(base, bytes), (int)off, 0, 0);
#endif
}
constexpr uint32_t kDropOffset = 0xFFFFFF00u;   // past any resource here (all are below 2^31 bytes)

// grid (nqt * H * nkt * B), nqt = Q-block tiles and nkt = key tiles of the longest sequence
template <int D, bool CAUSAL, typename T, int NU>
__global__ __launch_bounds__(256) void delta_s(const T* __restrict__ k, const float* __restrict__ muk,
                                               const uint16_t* __restrict__ muqs, float* __restrict__ ds,
                                               Geo g, int B, int nqt, int nkt, float k2) {
  constexpr int QT = 32 * NU;                          // Q blocks of the tile
  __shared__ DsSmem<D, QT> sm;
  constexpr int KS = D / 16;                            // 16-channel MFMA k-steps
  constexpr int ROW = DsSmem<D, QT>::ROW;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = g.H, Hkv = g.Hkv, G = H / Hkv;
  const int L = xcd_remap(blockIdx.x, nqt * H * nkt * B);
  int rest = L;
  const int qt = rest % nqt; rest /= nqt;
  const int gq = rest % G; rest /= G;
  const int kt = rest % nkt; rest /= nkt;
  const int b = rest % B, hk = rest / B;
  const int h = hk * G + gq;
  const Seq sq = g.seq(b);
  const int N = sq.n, nqb = seq_blocks(sq), Npad = nqb * BQ;
  const int q0 = qt * QT, k0 = kt * DS_KT;
  if (q0 >= nqb || k0 >= Npad) return;                 // beyond this sequence
  const int qlast = min(q0 + QT, nqb) - 1;
  if (CAUSAL && k0 >= (qlast + 1) * BQ) return;        // every row of the tile stops earlier

  // the tile's Q blocks' mu_Q parts (rows past the sequence repeat its last block and are never
  // stored) and mu_K -> LDS.  Their loads go out first, so the LDS fill waits for them alone
  // while this wave's key rows are still arriving.
  constexpr int CPQ = 3 * D / 8;                       // 16-byte chunks per Q block
  const uint16_t* aq = muqs + blocks_off(sq, H, h) * 3 * D;
  uint4 av[QT * CPQ / 256];
#pragma unroll
  for (int it = 0; it < QT * CPQ / 256; ++it) {
    const int c = it * 256 + tid;
    av[it] = *reinterpret_cast<const uint4*>(aq + (size_t)min(q0 + c / CPQ, nqb - 1) * 3 * D + (c % CPQ) * 8);
  }
  float4 mk = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid < D / 4) mk = *reinterpret_cast<const float4*>(muk + ((size_t)b * Hkv + hk) * D + 4 * tid);
  __builtin_amdgcn_sched_barrier(0);                   // keep these loads ahead of the key rows

  // this wave's key rows, all k-steps (rows past the sequence read its last row and count as
  // zero)
  const long long ts = g.st.kt;
  const T* kbase = k + b * g.st.kb + (long long)sq.tok0 * ts + hk * g.st.kh;
  const int j0 = k0 + 64 * w;                          // this wave's first key
  In8<T> kr[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kr[t][ks] = load8(kbase + (long long)min(j0 + 32 * t + r, N - 1) * ts + 16 * ks + 8 * hl);

#pragma unroll
  for (int it = 0; it < QT * CPQ / 256; ++it) {
    const int c = it * 256 + tid;
    *reinterpret_cast<uint4*>(sm.a + (c / CPQ) * ROW + (c % CPQ) * 16) = av[it];
  }
  if (tid < D / 4) *reinterpret_cast<float4*>(&sm.muk[4 * tid]) = mk;
  __syncthreads();
  if (j0 >= Npad || (CAUSAL && j0 >= (qlast + 1) * BQ)) return;   // no key of this wave is stored

  // A tile u (Q blocks q0 + 32 u ..) is live if it has a Q block that stores key j0.  Both tiles
  // are multiplied either way (a branch per tile would split the MFMA schedule); a dead one is
  // just not stored.
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int qa = q0 + 32 * u;
    live[u] = qa < nqb && (!CAUSAL || j0 < (min(qa + 31, nqb - 1) + 1) * BQ);
  }

  // the 2 x 2 tile products, one k-step at a time; TAIL: the wave holds keys j >= N, which
  // count as zero (only the last wave of a sequence takes that path)
  f32x16 acc[NU][2] = {};
  auto gemm = [&](auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 16 * ks + 8 * hl;                 // this lane's 8 channels of the k-step
      const float4 m0 = *reinterpret_cast<const float4*>(&sm.muk[c0]);
      const float4 m1 = *reinterpret_cast<const float4*>(&sm.muk[c0 + 4]);
      const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      bf16x8 A[NU][3];
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          A[u][p] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const s16x8*>(sm.a + (32 * u + r) * ROW + (p * D + c0) * 2));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = kr[t][ks].f(e) - mm[e];      // gamma_K, RN32
          xb[e] = TAIL && j0 + 32 * t + r >= N ? 0.f : x;
        }
        const Split3 Bv = split3(xb);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          f32x16 c = acc[u][t];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][2], Bv.p[0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][1], Bv.p[1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][0], Bv.p[2], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][1], Bv.p[0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][0], Bv.p[1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][0], Bv.p[0], c, 0, 0, 0);
          acc[u][t] = c;
        }
      }
    }
  };
  if (j0 + 64 > N) gemm(std::true_type{});
  else gemm(std::false_type{});

  // lane holds Q blocks q0 + 32 u + 8 a + 4 hl + e (a, e < 4) of key column j0 + 32 t + r.  The
  // stores go through one buffer resource over rows q0 .. qlast of this head: fewer than 2^31
  // bytes (at most 64 rows of at most 2^23 keys), so 32-bit offsets reach every element and
  // an element that is not stored (Q block past the sequence, key past a causal row) takes
  // an offset past the end.
  const size_t row0 = ds_row_offset(CAUSAL, q0, Npad);
  float* const dsr = ds + ds_off(sq, CAUSAL, h) + row0;
  const uint32_t span = (uint32_t)((ds_row_offset(CAUSAL, qlast + 1, Npad) - row0) * 4);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (!live[u]) continue;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qb = q0 + 32 * u + 8 * a4 + 4 * hl + e;
        // row qb's first element relative to row q0's (causal rows hold (qb + 1) * 128 keys)
        const uint32_t rel = CAUSAL ? 64u * (uint32_t)((qb - q0) * (qb + q0 + 1)) : (uint32_t)(qb - q0) * (uint32_t)Npad;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int j = j0 + 32 * t + r;
          const bool ok = qb < nqb && (!CAUSAL || (j >> 7) <= qb);
          store_or_drop(dsr, span, ok ? (rel + (uint32_t)j) * 4u : kDropOffset, acc[u][t][4 * a4 + e] * k2);
        }
      }
  }
}

// ---------------------------------------------------------------------------------------
// debug: internal layouts -> plain layouts
// ---------------------------------------------------------------------------------------
__global__ void copy_rows_i8(const int8_t* __restrict__ src, int8_t* __restrict__ dst, int heads, int N,
                             int Npad, int d, bool fp6) {
  const size_t total = (size_t)heads * N * d;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t hd = i / ((size_t)N * d), rem = i % ((size_t)N * d);
    const size_t r = rem / d;
    const int c = (int)(rem % d);
    const uint8_t* row = reinterpret_cast<const uint8_t*>(src) + (hd * Npad + r) * d;
    if (!fp6) {
      dst[i] = (int8_t)row[c];
    } else {                                   // unpack one E2M3 code and decode it
      const int bit = 6 * (c & 31);
      const uint8_t* slot = row + 32 * (c >> 5);
      const uint32_t b = ((uint32_t)slot[bit >> 3] | ((uint32_t)slot[(bit >> 3) + 1] << 8)) >> (bit & 7) & 63u;
      const int e = (b >> 3) & 3, m = b & 7;
      const int mag = e == 0 ? 0 : ((8 + m) << (e - 1)) >> 3;   // (1 + m/8) 2^(e-1), an integer here
      dst[i] = (int8_t)((b & 0x20) ? -mag : mag);
    }
  }
}
__global__ void copy_rows_f32(const float* __restrict__ src, float* __restrict__ dst, size_t rows, int n,
                              int npad, float mul) {
  const size_t total = rows * n;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / n, c = i % n;
    dst[i] = src[r * npad + c] * mul;
  }
}
// Delta_S rows -> [heads][nqb][N] in natural units; entries a causal row does not store are 0
__global__ void copy_ds(const float* __restrict__ src, float* __restrict__ dst, int heads, int nqb, int N, int Npad,
                        bool causal, float mul) {
  const size_t total = (size_t)heads * nqb * N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t hd = i / ((size_t)nqb * N);
    const int qb = (int)((i / N) % nqb), j = (int)(i % N);
    dst[i] = j < ds_row_len(causal, qb, Npad)
                 ? src[hd * ds_head_elems(causal, nqb, Npad) + ds_row_offset(causal, qb, Npad) + j] * mul
                 : 0.f;
  }
}
__global__ void expand_kscale(const float* __restrict__ kscale, float* __restrict__ dst, int heads, int N, int nkb) {
  const size_t total = (size_t)heads * N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t hd = i / N;
    const int j = (int)(i % N);
    dst[i] = kscale[(hd * nkb + j / BK) * 2 + ((j & 7) >> 2)];
  }
}
__global__ void unpermute_v(const uint8_t* __restrict__ vc, uint8_t* __restrict__ dst, int heads, int N, int Npad,
                            int d) {
  const size_t total = (size_t)heads * N * d;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t hd = i / ((size_t)N * d);
    const int j = (int)((i / d) % N), c = (int)(i % d);
    const int g = j / VGROUP, jj = j % VGROUP;
    const int pos = 32 * ((jj >> 2) & 1) + 16 * (jj >> 5) + 4 * ((jj >> 3) & 3) + (jj & 3);
    dst[i] = vc[((hd * (Npad / VGROUP) + g) * d + c) * VGROUP + pos];
  }
}

// the sequence table of a varlen batch, 64 entries per launch, passed by value
struct SeqChunk {
  Seq e[64];
  int first, count;
};
__global__ void write_seq_table(SeqChunk c, Seq* dst) {
  if ((int)threadIdx.x < c.count) dst[c.first + threadIdx.x] = c.e[threadIdx.x];
}

template <int D, typename T>
hipError_t launch_prologue_d(const Dims& Dm, const Ptrs& P, hipStream_t s) {
  const float R = Dm.qk_bits == 4 ? 7.f : 127.f;
  const Geo g = make_geo(Dm, P.seqs);
  const T* q = reinterpret_cast<const T*>(P.q);
  const T* k = reinterpret_cast<const T*>(P.k);
  const T* v = reinterpret_cast<const T*>(P.v);
  const int nkv = Dm.B * Dm.Hkv * D;
  init_stats<<<(nkv + 255) / 256, 256, 0, s>>>(P.ksum, P.vamax, nkv, Dm.bf16 ? kLimbs : 1);
  const dim3 gs((Dm.N + 255) / 256, Dm.B * Dm.Hkv), gq(Dm.nkb, Dm.B * Dm.Hkv);
  // INT4-range codes (R = 7) are stored as FP6: a compile-time switch of the code store
  auto kvq = [&](auto pv16, auto qk4) {
    kv_quant<D, decltype(pv16)::value, T, decltype(qk4)::value><<<gq, 256, 0, s>>>(
        k, v, P.ksum, P.vamax, P.kcodes, P.vcodes, P.kscale, P.muk, P.vscale, g, R);
  };
  const bool qk4 = Dm.qk_bits == 4;
  // statistics (K, and V unless it stays 16-bit) and the Q prologue: one launch
  const int nks = (int)(gs.x * gs.y), nsq = nks + Dm.nqb * Dm.B * Dm.H;
  auto sq = [&](auto vstats, auto q4) {
    stats_and_q<D, decltype(vstats)::value, T, decltype(q4)::value><<<nsq, 256, 0, s>>>(
        k, v, P.ksum, P.vamax, q, P.qcodes, P.qscale, P.muq, P.muqs, g, R, (int)gs.x, nks, Dm.nqb);
  };
  const bool vstats = Dm.pv_bits != 16;
  if (vstats) {
    if (qk4) sq(std::true_type{}, std::true_type{});
    else sq(std::true_type{}, std::false_type{});
  } else {
    if (qk4) sq(std::false_type{}, std::true_type{});
    else sq(std::false_type{}, std::false_type{});
  }
  if (Dm.pv_bits == 16) {
    if (qk4) kvq(std::true_type{}, std::true_type{});
    else kvq(std::true_type{}, std::false_type{});
  } else {
    if (qk4) kvq(std::false_type{}, std::true_type{});
    else kvq(std::false_type{}, std::false_type{});
  }
  const float k2 = (float)(1.4426950408889634 / sqrt((double)D));
  // 64 Q blocks per workgroup when sequences are long (the key split is shared by more MFMAs),
  // 32 when they are short on average (varlen prefill batches: less work on rows past the end)
  auto dsl = [&](auto nu) {
    constexpr int NU = decltype(nu)::value;
    const int nqt = (Dm.nqb + 32 * NU - 1) / (32 * NU), nkt = (Dm.Npad + DS_KT - 1) / DS_KT;
    const int gds = nqt * Dm.H * nkt * Dm.B;
    if (Dm.causal)
      delta_s<D, true, T, NU><<<gds, 256, 0, s>>>(k, P.muk, P.muqs, P.ds, g, Dm.B, nqt, nkt, k2);
    else
      delta_s<D, false, T, NU><<<gds, 256, 0, s>>>(k, P.muk, P.muqs, P.ds, g, Dm.B, nqt, nkt, k2);
  };
  if (Dm.tot_pad >= 48LL * BQ * Dm.B) dsl(std::integral_constant<int, 2>{});
  else dsl(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seq_table(const Seq* host, int n, Seq* dev, hipStream_t s) {
  for (int first = 0; first < n; first += 64) {
    SeqChunk c{};
    c.first = first;
    c.count = n - first < 64 ? n - first : 64;
    for (int i = 0; i < c.count; ++i) c.e[i] = host[first + i];
    write_seq_table<<<1, 64, 0, s>>>(c, dev);
  }
  return hipGetLastError();
}

hipError_t launch_prologue(const Dims& D, const Ptrs& P, hipStream_t s) {
  if (D.bf16) return D.d == 128 ? launch_prologue_d<128, __bf16>(D, P, s) : launch_prologue_d<64, __bf16>(D, P, s);
  return D.d == 128 ? launch_prologue_d<128, __half>(D, P, s) : launch_prologue_d<64, __half>(D, P, s);
}

hipError_t launch_debug_copy(const Dims& D, const Ptrs& P, hipStream_t s, float* mu_k, int8_t* k_codes,
                             float* k_scales, uint8_t* v_codes, float* v_scales, float* mu_q, int8_t* q_codes,
                             float* q_scales, float* delta_s_out) {
  const int hkv = D.B * D.Hkv, hq = D.B * D.H;
  const int grid = 1024, blk = 256;
  if (mu_k) {
    hipError_t e = hipMemcpyAsync(mu_k, P.muk, (size_t)hkv * D.d * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  const bool pv8 = D.pv_bits == 8;     // fp16 V has no codes or scales to copy
  if (v_scales && pv8) {
    hipError_t e = hipMemcpyAsync(v_scales, P.vscale, (size_t)hkv * D.d * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  if (mu_q) {
    hipError_t e = hipMemcpyAsync(mu_q, P.muq, (size_t)hq * D.nqb * D.d * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  const bool fp6 = D.qk_bits == 4;    // INT4-range codes are stored as packed FP6 E2M3
  if (k_codes) copy_rows_i8<<<grid, blk, 0, s>>>(P.kcodes, k_codes, hkv, D.N, D.Npad, D.d, fp6);
  if (q_codes) copy_rows_i8<<<grid, blk, 0, s>>>(P.qcodes, q_codes, hq, D.N, D.Npad, D.d, fp6);
  if (k_scales) expand_kscale<<<grid, blk, 0, s>>>(P.kscale, k_scales, hkv, D.N, D.nkb);
  if (q_scales) copy_rows_f32<<<grid, blk, 0, s>>>(P.qscale, q_scales, (size_t)hq, D.N, D.Npad, 1.f);
  if (v_codes && pv8) unpermute_v<<<grid, blk, 0, s>>>(P.vcodes, v_codes, hkv, D.N, D.Npad, D.d);
  if (delta_s_out) {
    const float inv_k2 = (float)(sqrt((double)D.d) / 1.4426950408889634);
    copy_ds<<<grid, blk, 0, s>>>(P.ds, delta_s_out, hq, D.nqb, D.N, D.Npad, D.causal != 0, inv_k2);
  }
  return hipGetLastError();
}

}  // namespace sage
