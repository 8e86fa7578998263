// Fused SageAttention2 attention kernel for gfx950 (CDNA4).
//
// Page "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and Per-thread
// INT4 Quantization" (mlsanity.com, arXiv 2411.10958), section "Abstract (arXiv)": QK^T on
// low-bit integer codes with thread-granular scales, P~ and V in FP8, two-level accumulation
// of P~V.  zhaifeiyue.github.io commentary on arXiv 2411.10958: the paper's Sec. 3.4 finds the
// FP8 matrix-instruction accumulator narrower than fp32 and accumulates each block locally
// before an fp32 global sum; per-thread scales must follow the matrix-instruction layout.
// pith.science verdict on arXiv 2505.21136, keys "key_machinery" (delta_P and per-channel
// delta_V; here the static delta_P = 1/P_r: every p = 2^(z - m) with the running maximum m is at
// most 1, so p * P_r never exceeds P_r) and "supporting_citations" (online softmax and
// FlashAttention tiling).
//
// Design (a group of 4 waves x 32 queries = the 128 queries of one Q block of one (b, h); a
// workgroup holds one group, or two that share every K/V tile, see attn_fwd):
//   * S^T = K Q^T on v_mfma_i32_32x32x32_i8 (the full-rate int8 shape on gfx950): A = K tile
//     from LDS, B = the wave's 32 query rows held in VGPRs for the whole KV loop.  Lane l owns
//     query column i = l % 32 and keys 8a + 4(l / 32) + r of every 32-key tile, so one
//     delta_Q * delta_K product dequantizes all of a lane's accumulators.
//   * The S^T accumulators already sit in the B-operand layout of v_mfma_f32_32x32x64_f8f6f4
//     (lane l: column l % 32, 32 consecutive k-slots): P~ goes from registers to the FP8 MFMA
//     with no LDS round trip; V^T is pre-permuted by the prologue into the same k-slot order.
//   * Two-level P~V accumulation: on gfx950 each FP8 MFMA sums its 64 products inside the
//     matrix unit with reduced precision (the block-local level, 64 keys), and adds that sum to
//     its C operand at fp32 precision (the global level).  So the fp32 output accumulator O is
//     itself the C operand: O <- O * alpha (skipped when the wave's running maxima did not
//     move), then O += P~ V per 64-key half.  The narrow sum never spans more than 64 products.
//   * K/V code tiles stream HBM -> LDS with direct-to-LDS buffer loads (buffer_load_dwordx4 lds),
//     in a ring of two stages (three at d = 64 in the FP8 mode, where a block's arithmetic is
//     too short to cover a tile issued only one block ahead), 16-byte chunks XOR-swizzled
//     against LDS bank conflicts.
//   * Workgroup ids are remapped so each XCD (own L2) works through whole kv heads (of every
//     sequence of the batch), with the query heads that share a kv head side by side for each
//     Q block; causal grids start with each sequence's longest (diagonal-most) query blocks.
//   * fp16 P V (PV16; the high-fidelity "qk_int8_pv_fp16" mode of the blog page "SageAttention：
//     大模型量化注意力加速实践指南", section on precision control): V stays fp16 and P = e^(z - m)
//     is rounded to fp16 into the B operand of v_mfma_f32_32x32x16_f16 (8 k-slots per lane: a
//     lane's keys 8a + 4(l / 32) + r of two adjacent a), accumulating straight into the fp32
//     output accumulator.  The fp16 V tile is twice the FP8 one, so it has one LDS stage: the
//     next block's V is issued once every wave is done with the current one and lands while
//     the next QK^T and softmax run.
#include <type_traits>

#include "sage_internal.h"

namespace sage {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

// The 16-bit float of the fp16 P V path: fp16, or bf16 for bf16 inputs (V keeps its input type)
template <bool BF> struct PV16T;
template <> struct PV16T<false> {
  typedef h8 v8;
  typedef h2 v2;
  static __device__ v16f mfma(v8 a, v8 b, v16f c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};
template <> struct PV16T<true> {
  typedef b8 v8;
  typedef b2 v2;
  static __device__ v16f mfma(v8 a, v8 b, v16f c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};

constexpr float kLog2Pr = 8.807354922057604f;   // log2(448)

// The row sum of P~ on v_mfma_f32_16x16x128_f8f6f4, with P~ as its B operand exactly as packed
// for the 32x32x64 P~V instruction.  Each group g = l / 16 of 16 lanes supplies one quarter of the
// k range for columns l % 16; in the 32x32x64 layout lane l holds query l % 32 and 32 keys, so
// groups 0 and 2 hold queries 0-15 (two key ranges each), groups 1 and 3 queries 16-31.  The A
// operand selects: its row r (lane r % 16 of group g supplies A[r][k] for that group's k range)
// is FP8 1.0 where r % 4 == 0 and (r / 4) % 2 == g % 2, else zero.  Then output row 4G of column
// n sums the lanes 16g + n with g = G (mod 2), i.e. all keys of query 16 (G % 2) + n, and that
// row is element 0 of the accumulator of lane 16 G + n -- the lane holding that query.  One
// 16x16x128 instruction per 64 keys (half the matrix time of a 32x32x64 against all-ones).
__device__ inline v8i rowsum_selector(int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int x = ((r & 3) == 0 && ((r >> 2) & 1) == (g & 1)) ? 0x38383838 : 0;
  return (v8i){x, x, x, x, x, x, x, x};
}
__device__ inline v4f rowsum_mfma(const v8i& sel, const v8i& pb, v4f acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pb, acc, 0, 0, 0, 0, 0, 0);
}

// O <- O * alpha before a block's P~V (or P V) matrix instructions accumulate into O.  alpha is
// per query (lane column); when no query of the wave raised its running maximum, every alpha is
// exactly 1 and the whole wave skips the multiplications (a wave-uniform branch).
template <int NT>
__device__ inline void rescale_o(v16f (&og)[NT], float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) == 0) return;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) og[ct][e] *= alpha;
}

struct AttnArgs {
  const int8_t* qcodes;
  const int8_t* kcodes;
  const uint8_t* vcodes;
  const float* qscale;
  const float* kscale;
  const float* vscale;
  const float* ds;
  __half* o;
  Geo g;                // sequences, strides; g.causal: Delta_S rows stored triangularly
  int B, nqb;           // sequences; Q blocks of the longest one
  float k2;             // log2(e) / sqrt(d)
  int dbg_b, dbg_h, dbg_qb, dbg_kb;
  int32_t* dbg_out;
};

// V stages: FP8 codes [64-key group][channel][64 slots], one per K stage; or fp16 V
// [16-key group][channel][16 slots], one stage.  16-byte chunks swizzled in both.
// GROUPS: Q blocks per workgroup (4 waves each) sharing every K/V tile; each has its Delta_S row.
template <int D, bool PV16, int GROUPS = 1>
struct Smem {
  // K (and FP8 V, Delta_S) stages: a ring of three at d = 64 in the FP8 mode, where a block's
  // arithmetic is short enough that a tile issued one block ahead can still be in flight
  static constexpr int NST = (!PV16 && D == 64) ? 3 : 2;
  static constexpr int VST = PV16 ? 1 : NST;
  __attribute__((aligned(16))) int8_t k[NST][BK * D];  // K tile rows, 16-byte chunks swizzled
  __attribute__((aligned(16))) uint8_t v[VST][BK * D * (PV16 ? 2 : 1)];
  __attribute__((aligned(16))) float ds[NST][GROUPS][BK];
};

// int32 S^T accumulators to floats, exactly (|S| <= 127^2 * 128 < 2^21).  At d = 128 they start
// from the bit pattern of the float 1.5 * 2^23, so after the MFMA adds S the bits read as the
// float 1.5 * 2^23 + S (same binade, unit spacing) and one fp32 subtraction yields S.  At d = 64
// they start from zero and v_cvt_f32_i32 converts them: in this kernel that measured 7 % faster
// than the subtraction at d = 64 and 5 % slower at d = 128.
template <int D> constexpr bool kCvtS = D == 64;
template <int D> constexpr int kAccInit = kCvtS<D> ? 0 : 0x4B400000;
constexpr float kAccBiasF = 12582912.0f;   // 1.5 * 2^23
// P~ V in two 64-key halves, each half's matrix instructions issued as soon as its P~ is packed,
// so they overlap the next half's exponentials.  At d = 128 it measured -5 % on a causal
// INT4-range workload and -1 to -1.5 % on INT8 ones; at d = 64 its 20 more live registers cost
// the third wave per SIMD (+5 %), so d = 64 keeps one pass.
template <int D> constexpr bool kSplitPV = D == 128;

template <int D>
__device__ inline float s_to_float(int acc) {
  return kCvtS<D> ? (float)acc : __int_as_float(acc) - kAccBiasF;
}

// XOR swizzles of the 16-byte chunk index inside an LDS row.  Each operand read has 32 lanes
// fetch 16 bytes from 32 consecutive rows (an aligned group of 32) at one logical chunk; the
// swizzles spread those rows over distinct bank groups whether the LDS serves 8 lanes per cycle
// over 32 banks or 16 lanes per cycle over 64 banks (the plain swizzle row & 7 left 2-way
// conflicts on gfx950).  None depends on the bits of the row above the 32-row group (row >> 5
// at d = 128), so the tile-load offsets of one lane differ by exactly 4 KB from one load
// instruction to the next and need a single register (see TileLoader).
template <int D>
__device__ inline int kswz(int row) {       // K rows: 128 bytes (d = 128) or 64 bytes (d = 64)
  return D == 128 ? ((row & 7) ^ ((row >> 3) & 3)) : (((row >> 1) ^ (row >> 3)) & 3);
}
__device__ inline int vswz(int c) {         // V^T rows: 64 bytes per channel
  return ((c >> 1) ^ (c >> 3)) & 3;
}
__device__ inline int v16swz(int c) {       // fp16 V^T rows: 32 bytes per channel and group
  return ((c >> 2) ^ (c >> 3)) & 1;
}

// combine a value with the one held by lane l ^ 32 (the other half holding the same query)
__device__ inline float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void;

// direct-to-LDS instructions per wave per tile: K codes (and FP8 V codes), fp16 V
template <int D>
constexpr int kTileInstrs = BK * D / 16 / 64 / WAVES;

// Tile loads: buffer loads straight to LDS (buffer_load_dwordx4 ... lds).  Each operand stream
// has a buffer resource over this (sequence, head)'s data; a lane's byte offset inside a tile is
// the same for every block, so it is computed once, and the block moves only the scalar
// offset.  (Per-lane 64-bit pointers advanced every block cost ~20 VALU instructions per block.)
// Loads past a resource's end return zeros (range-checked).
// The buffer builtins exist only for the GPU target: their code is compiled in the device pass
// (in the host pass, kernels using them otherwise lost their launch stubs without a diagnostic).

template <int D, bool PV16, int GROUPS = 1>
struct TileLoader {
  static constexpr int WT = WAVES * GROUPS;                 // waves that load each K/V tile
  static constexpr int NK = BK * D / 16 / 64 / WT;          // K (and FP8 V) instructions per wave
  static constexpr int NV = NK * (PV16 ? 2 : 1);
  static constexpr int VB = PV16 ? 2 : 1;                   // V bytes per element
  static constexpr int STEP = WT * 64 * 16;                 // bytes per load instruction and workgroup
  const void *kp, *vp, *dp;
  uint32_t kbytes, vbytes, dbytes;
  uint32_t koff, voff;   // this lane's offset for instruction m = 0; instruction m adds m * STEP

  // kc, vc: the head's K codes / V rows; dsrow: the wave's Q block's Delta_S row of ds_len
  // floats; wv: wave index in the workgroup
  __device__ TileLoader(const int8_t* kc, const uint8_t* vc, const float* dsrow, int nkb, int ds_len, int wv,
                        int lane) {
    kp = kc; kbytes = (uint32_t)nkb * BK * D;
    vp = vc; vbytes = (uint32_t)nkb * BK * D * VB;
    dp = dsrow; dbytes = (uint32_t)ds_len * 4;
    // 16-byte chunk p of the tile in LDS (instruction m, wave wv, lane) holds the global chunk of
    // row p / (chunks per row) at swizzled position: the LDS side of a load is linear in the lane
    constexpr int CPR = D / 16;                             // 16-byte chunks per K row
    const int p = wv * 64 + lane;
    const int row = p / CPR, pc = p % CPR;
    koff = (uint32_t)(row * D + ((pc ^ kswz<D>(row)) * 16));
    constexpr int RB = PV16 ? 32 : VGROUP;                  // bytes per V LDS row (group, channel)
    constexpr int CR = RB / 16;
    const int vrow = p / CR, vpc = p % CR;                  // vrow = group * D + channel
    const int sw = PV16 ? v16swz(vrow % D) : vswz(vrow % D);
    voff = (uint32_t)(vrow * RB + ((vpc ^ sw) * 16));
  }

  // K codes of block kb into stage st, and the wave's group's Delta_S row slice (each of the
  // group's 4 waves a quarter of it, so every wave issues the same number of loads per block).
  // The Delta_S load goes first, so a wait for "all but the last NK" loads leaves only K chunks
  // outstanding.  w: wave index in its group; gi: the group.
  template <class SM>
  __device__ void issue_k(SM& sm, int st, int kb, int wv, int w, int gi, int lane) const {
#if defined(__HIP_DEVICE_COMPILE__)
    if (lane < BK / 4 / WAVES)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(dp, dbytes), (lds_void*)(sm.ds[st][gi] + w * (BK / WAVES)), 16,
                                               lane * 16 + w * (BK / WAVES) * 4, kb * BK * 4, 0, 0);
    const auto kr = make_rsrc(kp, kbytes);
#pragma unroll
    for (int m = 0; m < NK; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(sm.k[st] + (m * WT + wv) * 1024), 16, koff,
                                               kb * BK * D + m * STEP, 0, 0);
#endif
  }

  // V of block kb into stage st: FP8 codes (64-byte rows) or 16-bit V (32-byte rows, twice the
  // instructions).
  template <class SM>
  __device__ void issue_v(SM& sm, int st, int kb, int wv) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto vr = make_rsrc(vp, vbytes);
#pragma unroll
    for (int m = 0; m < NV; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(sm.v[st] + (m * WT + wv) * 1024), 16, voff,
                                               kb * BK * D * VB + m * STEP, 0, 0);
#endif
  }
};

__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// wait until at most the loads of one block (its Delta_S slice, K and V tiles) are outstanding
template <int D>
__device__ inline void wait_all_but_one_block() {
  static_assert(2 * kTileInstrs<D> + 1 == 5, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
}

// wait until at most the last kTileInstrs<D> vector loads of this wave are outstanding
template <int D>
__device__ inline void wait_all_but_k_tile() {
  static_assert(kTileInstrs<D> == 4 || kTileInstrs<D> == 2, "vmcnt immediate");
  if (kTileInstrs<D> == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
}

// S^T tiles (32 keys each) x the wave's 32 queries, exact.  INT8 codes: v_mfma_i32_32x32x32_i8
// from kAccInit, 16 code bytes per lane per k-step.  INT4-range codes
// (stored as FP6 E2M3, 24 bytes of each 32-byte slot): v_mfma_f32_32x32x64_f8f6f4 in FP6 mode from
// zero, one slot per lane per k-step, at twice the INT8 rate; the products and sums of integers
// this small are exact in its accumulator, so S arrives as fp32.
template <int D, bool QK4, class SM>
__device__ inline void qk_tiles(const SM& sm, int st, const v4i (&qreg)[D / 32], int col, int half,
                                v16i (&sacc)[BK / 32]) {
#pragma unroll
  for (int t = 0; t < BK / 32; ++t) {
    const int row = 32 * t + col;
    if (QK4) {
      v16f acc = {};
#pragma unroll
      for (int s = 0; s < D / 64; ++s) {
        const int c0 = 4 * s + 2 * half;       // this lane's two 16-byte chunks of the 64-channel step
        const v4i lo = *reinterpret_cast<const v4i*>(sm.k[st] + row * D + (c0 ^ kswz<D>(row)) * 16);
        const v4i hi = *reinterpret_cast<const v4i*>(sm.k[st] + row * D + ((c0 + 1) ^ kswz<D>(row)) * 16);
        const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const v8i bv = {qreg[2 * s][0], qreg[2 * s][1], qreg[2 * s][2], qreg[2 * s][3],
                        qreg[2 * s + 1][0], qreg[2 * s + 1][1], qreg[2 * s + 1][2], qreg[2 * s + 1][3]};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 2, 2, 0, 0, 0, 0);   // FP6 E2M3
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[t][e] = __float_as_int(acc[e]);
    } else {
      constexpr int a0 = kAccInit<D>;
      v16i acc = {a0, a0, a0, a0, a0, a0, a0, a0, a0, a0, a0, a0, a0, a0, a0, a0};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const int pc = (2 * s + half) ^ kswz<D>(row);
        const v4i av = *reinterpret_cast<const v4i*>(sm.k[st] + row * D + pc * 16);
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, qreg[s], acc, 0, 0, 0);
      }
      sacc[t] = acc;
    }
  }
}

// GROUPS = 2 (FP8 mode, d = 128): one workgroup of 8 waves, two groups of 4, and every K/V tile is
// loaded once for both groups.  Non-causal: two Q blocks of the same (sequence, head).  A CU then
// holds one such workgroup instead of two independent ones, so its two Q blocks run in step and
// finish together (two independent workgroups on a CU finish at different times, the older one
// being served first, and the last one of a round then runs alone).  Causal (fixed-length GQA
// batches): the same Q block of two query heads of one kv head, whose work is identical, so the
// K/V tiles of a kv head are fetched once per pair of query heads.
template <int D, bool CAUSAL, bool DUMP, bool QK4, bool PV16, bool BF, int GROUPS>
__global__ __launch_bounds__(256 * GROUPS, GROUPS == 1 ? 2 : 1) void attn_fwd(AttnArgs a) {
  static_assert(GROUPS == 1 || (!PV16 && !DUMP && D == 128), "two groups per workgroup: FP8 mode, d = 128");
  typedef PV16T<BF> PT;
  __shared__ Smem<D, PV16, GROUPS> sm;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform: kept in a scalar
  const int gi = wv / WAVES, w = wv % WAVES;                 // Q-block group, wave in the group

  const int H = a.g.H, Hkv = a.g.Hkv;
  int b, h, qb;
  bool idle = false;                            // this group has no Q block
  Seq sq;
  if (DUMP) {
    b = a.dbg_b; h = a.dbg_h; qb = a.dbg_qb;
    sq = a.g.seq(b);
  } else if (GROUPS == 2 && CAUSAL) {
    // query-head pairs, in the order below with pairs in place of single heads
    const int G = H / Hkv, pairs = G / 2;
    const int total = a.B * (H / 2) * a.nqb;
    const int L = xcd_remap(blockIdx.x, total);
    const int pr = L % pairs, r = L / pairs;
    const int qi = r % a.nqb, kbi = r / a.nqb;
    b = kbi % a.B;
    h = (kbi / a.B) * G + 2 * pr + gi;
    sq = a.g.seq(b);
    qb = seq_blocks(sq) - 1 - qi;               // longest rows first
  } else {
    // kv-head-major order: each XCD's contiguous share holds whole kv heads of every sequence,
    // so varlen batches split evenly and a kv head's codes stay in one XCD's L2; within it the
    // query heads sharing the kv head come together for each Q block, so they stream the same
    // K/V tiles at the same time
    const int nq = (a.nqb + GROUPS - 1) / GROUPS;            // workgroups per (sequence, head)
    const int total = a.B * H * nq, G = H / Hkv;
    const int L = xcd_remap(blockIdx.x, total);
    const int g = L % G, r = L / G;
    const int qi = r % nq, kbi = r / nq;
    b = kbi % a.B;
    h = (kbi / a.B) * G + g;
    sq = a.g.seq(b);
    const int sb = seq_blocks(sq);
    if (qi * GROUPS >= sb) return;              // beyond this sequence (varlen)
    // this group's Q block; a second group past the sequence's end repeats group 0's block in
    // step with it (loading its share of the tiles, meeting the barriers) and stores nothing
    const int qx = qi * GROUPS + gi;
    idle = qx >= sb;
    qb = idle ? qi * GROUPS : (CAUSAL ? sb - 1 - qx : qx);
  }
  const int hk = h / (H / Hkv);
  const int N = sq.n, nkb = seq_blocks(sq);
  const int il = w * QW + col;                  // query within the block
  const int i = qb * BQ + il;                   // query within the sequence
  // this (sequence, head)'s workspace sections
  const size_t qrows = rows_off(sq, H, h), krows = rows_off(sq, Hkv, hk);
  const int8_t* kc = a.kcodes + krows * D;
  const uint8_t* vc = a.vcodes + krows * D * (PV16 ? 2 : 1);
  const float* kscl = a.kscale + blocks_off(sq, Hkv, hk) * 2;
  const float* dsrow = a.ds + ds_off(sq, a.g.causal, h) + ds_row_offset(a.g.causal, qb, nkb * BK);
  const TileLoader<D, PV16, GROUPS> ld(kc, vc, dsrow, nkb, ds_row_len(a.g.causal, qb, nkb * BK), wv, lane);

  // the wave's 32 query rows as the B operand of S^T = K Q^T (16 bytes per k-step)
  // (INT4 range: 32 bytes per 64-channel step, held as two consecutive v4i)
  v4i qreg[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const int ch = QK4 ? 64 * (s >> 1) + 32 * half + 16 * (s & 1) : 32 * s + 16 * half;
    qreg[s] = *reinterpret_cast<const v4i*>(a.qcodes + (qrows + i) * D + ch);
  }
  const float qd = a.qscale[qrows + i];

  if (DUMP) {
    ld.issue_k(sm, 0, a.dbg_kb, wv, w, 0, lane);
    wait_loads();
    __syncthreads();
    v16i sacc[BK / 32];
    qk_tiles<D, QK4>(sm, 0, qreg, col, half, sacc);
#pragma unroll
    for (int t = 0; t < BK / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jl = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
        a.dbg_out[il * BK + jl] = QK4 ? (int32_t)__int_as_float(sacc[t][e]) : (int32_t)s_to_float<D>(sacc[t][e]);
      }
    return;
  }

  const int nblk = CAUSAL ? qb + 1 : nkb;       // KV blocks of this Q block (both groups: nkb)
  float m_run = -INFINITY, l_part = 0.f;
  v16f og[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) og[ct] = (v16f){};
  const v8i rsel = rowsum_selector(lane);     // A operand of the P~ row-sum instruction

  constexpr int NST = Smem<D, PV16, GROUPS>::NST;
  // blocks 0 .. NST - 2 into stages 0 .. NST - 2; wait for block 0
  for (int i = 0; i < NST - 1 && i < nblk; ++i) {
    ld.issue_v(sm, i, i, wv);
    ld.issue_k(sm, i, i, wv, w, gi, lane);
  }
  if constexpr (NST == 3) {
    if (nblk > 1) wait_all_but_one_block<D>();
    else wait_loads();
  } else {
    wait_loads();
  }
  __syncthreads();
  int st = 0;                                   // stage of block kb: kb % NST

  // One KV block of this wave's group: S^T on the int8 MFMA, dequantize + bias (+ mask), online
  // softmax, P~ V on the FP8 MFMA (or P V on the fp16 MFMA).  MASK is set only for the causal
  // diagonal block.
  auto block = [&](const int kb, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const bool more = kb + 1 < nblk;

    v16i sacc[BK / 32];
    qk_tiles<D, QK4>(sm, st, qreg, col, half, sacc);

    // dequantize and add the Q-smoothing bias, in the log2 domain
    // both lane halves' delta_K through one wave-uniform (scalar) load, so that waiting for it
    // does not also wait for the tile prefetch just issued
    typedef __attribute__((address_space(4))) const float cfloat;   // read-only here: scalar load
    const cfloat* kdp = (const cfloat*)(kscl + kb * 2);
    const float kd0 = kdp[0], kd1 = kdp[1];
    const float kd = half ? kd1 : kd0;
    const float cmul = qd * kd * a.k2;
    float z[BK / 32][16];
    // the row max in two chains of three-input maxima (v_max3_f32: two new elements per
    // instruction); a max is exact in any order
    float mloc = -INFINITY, mloc2 = -INFINITY;
#pragma unroll
    for (int t = 0; t < BK / 32; ++t) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int j0 = 32 * t + 8 * qq + 4 * half;
        // read as an int vector: this stage was filled and waited for in the previous block
        const v4i dsv = *reinterpret_cast<const v4i*>(&sm.ds[st][gi][j0]);
        const float dsa[4] = {__int_as_float(dsv[0]), __int_as_float(dsv[1]), __int_as_float(dsv[2]), __int_as_float(dsv[3])};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sf = QK4 ? __int_as_float(sacc[t][4 * qq + r])                // exact S
                               : s_to_float<D>(sacc[t][4 * qq + r]);      // exact
          float x = fmaf(sf, cmul, dsa[r]);
          if (MASK) {
            const int j = kb * BK + j0 + r;
            if ((CAUSAL && j > i) || j >= N) x = -INFINITY;
          }
          z[t][4 * qq + r] = x;
        }
        mloc = fmaxf(fmaxf(mloc, z[t][4 * qq]), z[t][4 * qq + 1]);
        mloc2 = fmaxf(fmaxf(mloc2, z[t][4 * qq + 2]), z[t][4 * qq + 3]);
      }
    }
    // row max across the two lane halves holding the same query
    mloc = xhalf_max(fmaxf(mloc, mloc2));
    const float m_new = fmaxf(m_run, mloc);
    // a row has a finite max from its first block on (key 0 is never masked); the guards only
    // keep -inf - -inf out of the arithmetic
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    // p * P_r = 2^(z - mo) (FP8 P~); p = 2^(z - mo) (fp16 P)
    const float mo = (m_new == -INFINITY ? 0.f : m_new) - (PV16 ? 0.f : kLog2Pr);
    m_run = m_new;

    if (PV16) {
      // this block's fp16 V (issued at the end of the previous block) must have landed; later
      // loads (the next K tile) may still be in flight
      if (more) wait_all_but_k_tile<D>();
      else wait_loads();
      __syncthreads();
      rescale_o(og, alpha);

      // per 32-key tile: P = RN16(p) packed straight into two fp16 MFMA B operands (operand m
      // takes the lane's keys of accumulator quads 2m and 2m + 1), then P V into the fp32
      // output accumulator
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < BK / 32; ++t) {
        typename PT::v8 pb[2];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float p0 = __builtin_amdgcn_exp2f(z[t][4 * qq + 0] - mo);
          const float p1 = __builtin_amdgcn_exp2f(z[t][4 * qq + 1] - mo);
          const float p2 = __builtin_amdgcn_exp2f(z[t][4 * qq + 2] - mo);
          const float p3 = __builtin_amdgcn_exp2f(z[t][4 * qq + 3] - mo);
          lsum += (p0 + p1) + (p2 + p3);
          const typename PT::v2 lo = __builtin_convertvector((f2){p0, p1}, typename PT::v2);
          const typename PT::v2 hi = __builtin_convertvector((f2){p2, p3}, typename PT::v2);
          const int o = 4 * (qq & 1);
          pb[qq >> 1][o + 0] = lo[0];
          pb[qq >> 1][o + 1] = lo[1];
          pb[qq >> 1][o + 2] = hi[0];
          pb[qq >> 1][o + 3] = hi[1];
        }
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const int c = 32 * ct + col;
          const int hc = (half ^ v16swz(c)) * 16;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const typename PT::v8 va = *reinterpret_cast<const typename PT::v8*>(sm.v[0] + ((2 * t + m) * D + c) * 32 + hc);
            og[ct] = PT::mfma(va, pb[m], og[ct]);
          }
        }
        // keep the scheduler from hoisting later tiles' V reads (registers) above this one
        __builtin_amdgcn_sched_barrier(0);
      }
      l_part = fmaf(l_part, alpha, lsum);
      return;
    }

    // O * alpha first: the P~V matrix instructions below accumulate into O
    rescale_o(og, alpha);
    if constexpr (kSplitPV<D>) {
      // P~ = E4M3(p * P_r), packed straight into the FP8 MFMA B operand, one 64-key half (u) at a
      // time: the matrix instructions of half u -- its row sum, and its P~ V into O -- do not
      // depend on the exponentials of the next half, so the two interleave.
      v4f ls = {};
#pragma unroll
      for (int u = 0; u < BK / 64; ++u) {
        v8i pb;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * u + tt;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float p0 = __builtin_amdgcn_exp2f(z[t][4 * qq + 0] - mo);
            const float p1 = __builtin_amdgcn_exp2f(z[t][4 * qq + 1] - mo);
            const float p2 = __builtin_amdgcn_exp2f(z[t][4 * qq + 2] - mo);
            const float p3 = __builtin_amdgcn_exp2f(z[t][4 * qq + 3] - mo);
            // the first convert writes the low half; passing p0's (dead) bits as the untouched high
            // half saves materialising a zero register per word
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
            pb[tt * 4 + qq] = word;
          }
        }
        // the row sum of the weights that multiply V (P~ in FP8 units)
        ls = rowsum_mfma(rsel, pb, ls);
        // O += P~ V over this half's 64 keys, every channel tile
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const int c = 32 * ct + col;
          const uint8_t* row = sm.v[st] + (u * D + c) * VGROUP;
          const int sw = vswz(c);
          const v4i lo = *reinterpret_cast<const v4i*>(row + ((2 * half) ^ sw) * 16);
          const v4i hi = *reinterpret_cast<const v4i*>(row + ((2 * half + 1) ^ sw) * 16);
          const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          og[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, og[ct], 0, 0, 0, 0, 0, 0);
        }
      }
      l_part = fmaf(l_part, alpha, ls[0]);
    } else {
      // P~ = E4M3(p * P_r), packed straight into the FP8 MFMA B operand
      v8i pb[BK / 64];
#pragma unroll
      for (int t = 0; t < BK / 32; ++t) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float p0 = __builtin_amdgcn_exp2f(z[t][4 * qq + 0] - mo);
          const float p1 = __builtin_amdgcn_exp2f(z[t][4 * qq + 1] - mo);
          const float p2 = __builtin_amdgcn_exp2f(z[t][4 * qq + 2] - mo);
          const float p3 = __builtin_amdgcn_exp2f(z[t][4 * qq + 3] - mo);
          // the first convert writes the low half; passing p0's (dead) bits as the untouched high
          // half saves materialising a zero register per word
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
          pb[t >> 1][(t & 1) * 4 + qq] = word;
        }
      }
      // the row sum of the weights that multiply V (P~ in FP8 units)
      {
        v4f ls = {};
#pragma unroll
        for (int u = 0; u < BK / 64; ++u) ls = rowsum_mfma(rsel, pb[u], ls);
        l_part = fmaf(l_part, alpha, ls[0]);
      }

      // O += P~ V, 64 keys per matrix instruction
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) {
        const int c = 32 * ct + col;
#pragma unroll
        for (int u = 0; u < BK / 64; ++u) {
          const uint8_t* row = sm.v[st] + (u * D + c) * VGROUP;
          const int sw = vswz(c);
          const v4i lo = *reinterpret_cast<const v4i*>(row + ((2 * half) ^ sw) * 16);
          const v4i hi = *reinterpret_cast<const v4i*>(row + ((2 * half + 1) ^ sw) * 16);
          const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          og[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb[u], og[ct], 0, 0, 0, 0, 0, 0);
        }
      }
    }

  };

  // One step of the workgroup's stream of blocks: the loads of block kb + NST - 1, block kb
  // (MODE 0: unmasked, 1: the masked causal diagonal), then the wait for block kb + 1 and the
  // barrier.  Every wave loads its share of each tile and meets every barrier.
  auto step = [&](const int kb, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    // block kb + NST - 1 into the stage block kb - 1 used (every wave is past its barrier)
    const int stn = st == 0 ? NST - 1 : st - 1;
    const bool issue = kb + NST - 1 < nblk;
    if (issue) {
      if (!PV16) ld.issue_v(sm, stn, kb + NST - 1, wv);
      ld.issue_k(sm, stn, kb + NST - 1, wv, w, gi, lane);
    }
    block(kb, std::integral_constant<bool, MODE == 1>{});
    // block kb + 1 has landed (the loads issued above, for block kb + NST - 1, may still fly)
    if constexpr (NST == 3) {
      if (issue) wait_all_but_one_block<D>();
      else wait_loads();
    } else {
      wait_loads();
    }
    __syncthreads();
    // fp16 V has one stage: the next block's goes out once every wave is done with this one
    if (PV16 && kb + 1 < nblk) ld.issue_v(sm, 0, kb + 1, wv);
    st = st + 1 == NST ? 0 : st + 1;
  };
  typedef std::integral_constant<int, 0> Full;
  typedef std::integral_constant<int, 1> Diag;
  // the last block is masked when causal (the diagonal block); keys past N carry a Delta_S of
  // -inf, so a ragged tail needs no mask
  const int nfull = CAUSAL ? nblk - 1 : nblk;
  for (int kb = 0; kb < nfull; ++kb) step(kb, Full{});
  if (CAUSAL) step(nblk - 1, Diag{});

  // epilogue: O = acc * delta_V / l   (FP8: l sums P~, so it carries the 1/P_r, and the row-sum
  // instruction has already added both lane halves; fp16: no V scale, per-lane partial sums)
  const float l = PV16 ? xhalf_sum(l_part) : l_part;
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if (!idle && i < N) {
    __half* orow = a.o + b * a.g.st.qb + (long long)(sq.tok0 + i) * a.g.st.qt + h * a.g.st.qh;
    const float* vs = a.vscale + ((size_t)b * Hkv + hk) * D;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c0 = 32 * ct + 8 * qq + 4 * half;
        const float4 sc = PV16 ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(vs + c0);
        const float y0 = og[ct][4 * qq + 0] * sc.x * inv_l, y1 = og[ct][4 * qq + 1] * sc.y * inv_l;
        const float y2 = og[ct][4 * qq + 2] * sc.z * inv_l, y3 = og[ct][4 * qq + 3] * sc.w * inv_l;
        uint2 pk;                               // RNE to the output type (the input type)
        if (BF) {
          const b2 lo = __builtin_convertvector((f2){y0, y1}, b2), hi = __builtin_convertvector((f2){y2, y3}, b2);
          pk = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        } else {
          const h2 lo = __builtin_convertvector((f2){y0, y1}, h2), hi = __builtin_convertvector((f2){y2, y3}, h2);
          pk = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
        *reinterpret_cast<uint2*>(orow + c0) = pk;
      }
    }
  }
}

AttnArgs make_args(const Dims& D, const Ptrs& P) {
  AttnArgs a{};
  a.g = make_geo(D, P.seqs);
  a.B = D.B;
  a.nqb = D.nqb;
  a.qcodes = P.qcodes;
  a.kcodes = P.kcodes;
  a.vcodes = P.vcodes;
  a.qscale = P.qscale;
  a.kscale = P.kscale;
  a.vscale = P.vscale;
  a.ds = P.ds;
  a.o = P.o;
  a.k2 = (float)(1.4426950408889634 / sqrt((double)D.d));
  return a;
}

template <int DD, bool QK4, bool PV16, bool BF>
hipError_t launch_d(const Dims& D, const AttnArgs& a, hipStream_t s) {
  // FP8 mode at d = 128, non-causal: two Q blocks per workgroup sharing every K/V tile (causal
  // Q-block pairs measured slower: the second block is one shorter and idles on the last one)
  if constexpr (!PV16 && DD == 128) {
    if (!D.causal)
      return launch(attn_fwd<DD, false, false, QK4, PV16, BF, 2>, dim3(D.B * D.H * ((D.nqb + 1) / 2)), dim3(512), s, a);
    // causal GQA with an even number of query heads per kv head, fixed-length batches (in varlen
    // batches the pairs measured slower): two query heads of a kv head per workgroup
    if (!D.varlen && (D.H / D.Hkv) % 2 == 0)
      return launch(attn_fwd<DD, true, false, QK4, PV16, BF, 2>, dim3(D.B * (D.H / 2) * D.nqb), dim3(512), s, a);
  }
  const int grid = D.B * D.H * D.nqb;
  if (D.causal) return launch(attn_fwd<DD, true, false, QK4, PV16, BF, 1>, dim3(grid), dim3(256), s, a);
  return launch(attn_fwd<DD, false, false, QK4, PV16, BF, 1>, dim3(grid), dim3(256), s, a);
}

template <bool QK4, bool PV16>
hipError_t launch_qp(const Dims& D, const AttnArgs& a, hipStream_t s) {
  if (D.bf16) return D.d == 128 ? launch_d<128, QK4, PV16, true>(D, a, s) : launch_d<64, QK4, PV16, true>(D, a, s);
  return D.d == 128 ? launch_d<128, QK4, PV16, false>(D, a, s) : launch_d<64, QK4, PV16, false>(D, a, s);
}

}  // namespace

hipError_t launch_attention(const Dims& D, const Ptrs& P, hipStream_t s) {
  const AttnArgs a = make_args(D, P);
  if (D.pv_bits == 16) return D.qk_bits == 4 ? launch_qp<true, true>(D, a, s) : launch_qp<false, true>(D, a, s);
  return D.qk_bits == 4 ? launch_qp<true, false>(D, a, s) : launch_qp<false, false>(D, a, s);
}

hipError_t launch_qk_tile(const Dims& D, const Ptrs& P, int b, int h, int qb, int kb, int32_t* out, hipStream_t s) {
  AttnArgs a = make_args(D, P);
  a.dbg_b = b; a.dbg_h = h; a.dbg_qb = qb; a.dbg_kb = kb; a.dbg_out = out;
  const dim3 one(1), blk(256);
  if (D.qk_bits == 4)
    return D.d == 128 ? launch(attn_fwd<128, false, true, true, false, false, 1>, one, blk, s, a)
                      : launch(attn_fwd<64, false, true, true, false, false, 1>, one, blk, s, a);
  return D.d == 128 ? launch(attn_fwd<128, false, true, false, false, false, 1>, one, blk, s, a)
                    : launch(attn_fwd<64, false, true, false, false, false, 1>, one, blk, s, a);
}

}  // namespace sage
