// Receiver side: fused dequantize of P shards' messages and fp32 sum.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Inference
// bullet (after communication every tensor is converted back and the
// devices' values are summed). With one BF16 set per shard (a reading of the
// Selection bullet, whose ranges are per device) a feature's slot differs
// from shard to shard; the same kernels serve both forms.
//
// Window kernel (the fast path). A wave-tile is 512 consecutive features,
// 8 per lane, so each lane writes its 8 outputs of a token row as 32
// contiguous bytes of y (16 for bf16 output) and the wave writes 2 KB of
// whole cache lines. A 256-thread block takes 4 adjacent tiles of one block
// of token rows; all blocks of a row block run on one XCD (xcd_unit_block).
//  0. Setup, once per wave. The lane loads its 8 features' map entries, and
//     each shard's scales and zero points, with contiguous loads. Two scalar
//     map reads give the tile's code span and BF16 index runs, so the first
//     kR token rows are issued right behind those loads. A shard's int4
//     features among the 8 take consecutive slots, so all their codes lie in
//     the 8 bytes at the 4-byte aligned offset `cb` at or below the first
//     one's byte; two byte selectors (v_perm_b32) place each code's byte
//     under its feature, and a mask keeps its nibble. The selectors and masks
//     follow from the lane's 8-bit int4 mask and the first code's nibble, and
//     are computed four features per instruction. Each feature starts
//     from the constant -sum_p z*s over its int4 shards, and a high nibble,
//     kept in place as 16q, meets its scale divided by 16 (exact). The setup
//     is written with selects throughout: every lane runs the same
//     instructions, with no per-lane branches.
//  1. Per token row and shard, the tile's code span (at most 66 dwords) is
//     one coalesced 8-byte load on the first 33 lanes, so every packed byte
//     is requested once; the span goes through the wave's LDS stage, where
//     each lane reads its 8-byte window. (Loading the overlapping windows
//     straight from memory requests most bytes twice, and measured about
//     15% slower.) Each term is one v_fma_mix_f32: the code as an f16
//     denormal times the scale held multiplied by 2^24 (per-shard sets: a
//     byte-to-float conversion and an fma), bit for bit the same result.
//  2. BF16 values: the tile's entries of every shard (a contiguous run of
//     each shard's outlier block) ride in kOR registers across the wave,
//     loaded coalesced. They are written to a per-wave LDS table with one
//     row of P floats per feature that is BF16 on some shard (zeros where
//     it is int4), and the lane that owns the feature adds its row in shard
//     order from +0: no atomics, so the order is fixed by construction. A
//     feature BF16 on every shard has no int4 term, so its output is that
//     sum exactly. The sum reaches its feature through a select, so no other
//     feature sees it (not even a non-finite one). A tile with more entries
//     than the registers hold recomputes its BF16 features after the row
//     loop, term by term.
//  3. Shard groups (one set, fp32 output): more than 8 shards, or a message
//     past 2^31 bytes, run the window kernel once per group of shards, in
//     shard order. A later group (kAcc) loads each row's y with its codes and
//     continues every feature from it, BF16 sums included, so their shard
//     order from +0 holds across groups.
//
// General kernel: one thread per (token, feature). It evaluates each term as
// fl(q - z) * s, or the BF16 value, and adds the terms in shard order from
// +0, for any P, H, k, pitch and alignment.
#include <limits.h>

#include "common.hpp"

namespace btq {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kDqWaves = 4;
constexpr int kWinFeat = 8;                    // features per lane
constexpr int kWinTile = kWave * kWinFeat;     // 512 features per wave-tile
// Token rows in flight per wave. Two rows (with 2-3 waves per SIMD) keep
// HBM as busy as four, and measured up to 7% faster at large batches: fewer
// requests in flight per CU, and fewer registers.
constexpr int kDqRing = 2;
// Rows per wave: about 2048 waves (two per SIMD) when that leaves each wave
// at least dq_min_rows_two rows, else about 1024 (one per SIMD); up to 64
// rows. Two waves of 16 rows took large prefill at T=2048 from 28.7 to
// 26.5 us. Below 16 rows the fp32 receiver's setup costs more than the
// second wave hides; the bf16-output and per-shard receivers gain down to 8
// (7B prefill, T=2048: bf16 21.9 -> 18.9 us, per-shard 29.1 -> 28.2 us).
constexpr int64_t kDqWavesTwo = 2048;
constexpr int64_t kDqWavesOne = 1024;
__host__ __device__ constexpr int64_t dq_min_rows_two(bool per_shard, bool bf16_out) {
  return (per_shard || bf16_out) ? 8 : 16;
}

// fp32 -> bf16, round to nearest even, two values per instruction
// (v_cvt_pk_bf16_f32): a in the low half, b in the high half.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return (uint16_t)(bf16_pair(f, 0.0f) & 0xFFFFu); }

// Byte 0 of v in all four bytes (v_perm_b32: selector 0 picks byte 0 of the
// second operand).
__device__ __forceinline__ uint32_t splat_byte0(uint32_t v) { return __builtin_amdgcn_perm(0u, v, 0u); }

// fma(c, s, acc) with the code c given as an f16 denormal, c * 2^-24, in
// the low (fma_h0) or high (fma_h1) half of h, and s already multiplied by
// 2^24: the product is exactly c times the true scale, and the sum is
// rounded once, so the result is bit for bit that of fmaf((float)c, scale,
// acc). One instruction per term (v_fma_mix_f32) in place of a byte
// conversion and an fma; the compiler does not form it by itself.
__device__ __forceinline__ float fma_h0(uint32_t h, float s24, float acc) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(s24), "v"(acc));
  return d;
}
__device__ __forceinline__ float fma_h1(uint32_t h, float s24, float acc) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=v"(d)
      : "v"(h), "v"(s24), "v"(acc));
  return d;
}
constexpr float kTwo24 = 16777216.0f;
// v_perm selectors that spread bytes 0, 1 (or 2, 3) of a dword to the low
// bytes of its two 16-bit halves, with zero high bytes
constexpr uint32_t kSpread01 = 0x0C010C00u;
constexpr uint32_t kSpread23 = 0x0C030C02u;

// v[eu] (0 when eu is past the end), by selects.
template <int N>
__device__ __forceinline__ float pick8(const float (&v)[N], int eu) {
  float r = 0.0f;
#pragma unroll
  for (int e = 0; e < N; ++e) r = (e == eu) ? v[e] : r;
  return r;
}

// Marks a wave-uniform value as redefined here, in a scalar register (an
// empty asm): its load must be complete at this point, and cannot be moved
// below it.
template <typename V>
__device__ __forceinline__ void settle_s(V& v) {
  asm volatile("" : "+s"(v));
}

// Wave-wide counts from ballots (no LDS round trips): v in [0, 15] per lane.
__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}
__device__ __forceinline__ int wave_sum16(int v) {
  int s = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) s += __popcll(__ballot((v >> b) & 1)) << b;
  return s;
}
__device__ __forceinline__ int wave_prefix16(int v, int lane) {   // sum over lanes below
  const uint64_t below = lanes_below(lane);
  int s = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) s += __popcll(__ballot((v >> b) & 1) & below) << b;
  return s;
}
__device__ __forceinline__ int wave_max8(int v) {   // v in [0, 8]
  int m = 0;
#pragma unroll
  for (int u = 1; u <= 8; ++u) m = __ballot(v >= u) ? u : m;
  return m;
}

// Stage of one row's code spans, at the start of the wave's LDS: span dword
// d of shard p at d*kSP + 2p, kSP = 2*NP + 1. A lane's window of every shard
// is then two dwords at offsets 2p and 2p + kSP from one base, which the
// instructions carry (no per-row address arithmetic); no two shards' dwords
// are adjacent, so the compiler does not fuse writes that would need their
// registers paired; the odd stride keeps the window reads free of bank
// conflicts, and the span writes conflict at most 2 ways. Every lane writes
// its 8 bytes (the first 33 lanes the tile's span of at most 66 dwords).
constexpr int kStageLanes = 33;
__host__ __device__ constexpr int stage_stride(int np) { return 2 * np + 1; }

// LDS per wave of the window kernel, in dwords: the stage of one row's code
// spans (first, so that the window reads' offsets fit their instructions),
// the BF16 table (one row of NP floats per BF16 feature of the tile, at most
// kOR*64 entries), the entry -> table-row map of per-shard sets (kOR*64
// ints), one private dummy dword per lane for entries past the tile's count,
// and for fp32 output the 2 KB row that turns the lanes' 32-byte runs into
// whole-line stores.
template <int NP, int kOR, bool kPs>
__host__ __device__ constexpr int win_tab_dwords() { return kPs ? NP * kOR * kWave : kOR * kWave; }
__host__ __device__ constexpr int win_stage_dwords(int np) { return 2 * kWave * stage_stride(np); }
template <int NP, int kOR, bool kPs, bool kBf>
__host__ __device__ constexpr int win_lds_dwords() {
  return win_stage_dwords(NP) + win_tab_dwords<NP, kOR, kPs>() + (kPs ? kOR * kWave : 0) +
         kWave + (kBf ? 0 : kWinTile);
}

// NP: shards (1..8). kOR: BF16 entry registers per row (0: k = 0, no BF16
// entries to load). kR: ring depth.
// kPs: fmap is [P,H] (one set per shard) instead of [H]. kBf: y is bf16.
// Waves per SIMD the register budget aims at: 3 (at most 168 registers) for
// one set with two entry registers, else 2 (at most 256).
template <int NP, int kOR, int kR, bool kPs, bool kBf, bool kAcc>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu((!kPs && kOR <= 2 && !kAcc) ? 3 : 2)))
void dq_window_kernel(
    const uint8_t* __restrict__ packed, int pitch, const uint16_t* __restrict__ outl, int64_t T,
    int H, int k, int ntiles, int rows_per_wave, int64_t nrowblk, const float* __restrict__ scale,
    const uint8_t* __restrict__ zp, const int32_t* __restrict__ fmap, void* __restrict__ y) {
  constexpr int NM = kPs ? NP : 1;             // maps
  constexpr uint32_t kYB = kBf ? 2u : 4u;      // bytes per y value
  static_assert(!kAcc || !kBf, "shard groups: fp32 output");
  constexpr int kLds = win_lds_dwords<NP, kOR, kPs, kBf>();
  constexpr int kSP = stage_stride(NP);
  extern __shared__ __align__(16) float dq_smem[];
  int64_t rb, sub;
  const int ntgrp = (ntiles + kDqWaves - 1) / kDqWaves;
  if (!xcd_unit_block(blockIdx.x, ntgrp, nrowblk, &rb, &sub)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = (int)sub * kDqWaves + wave;
  if (c >= ntiles) return;   // past the last tile (no block barrier below)
  const int f0 = c * kWinTile;
  const int h0 = f0 + kWinFeat * lane;
  const bool active = h0 < H;   // H is a multiple of 8: a lane is all in or all out
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min(T - t0, (int64_t)rows_per_wave);   // >= 1
  uint32_t* const stage = reinterpret_cast<uint32_t*>(dq_smem + (size_t)wave * kLds);
  float* const tab = dq_smem + (size_t)wave * kLds + win_stage_dwords(NP);
  int* const inv = reinterpret_cast<int*>(tab + win_tab_dwords<NP, kOR, kPs>());
  float* const dummy = tab + win_tab_dwords<NP, kOR, kPs>() + (kPs ? kOR * kWave : 0);
  float* const yrow = dummy + kWave;   // fp32 output only

  // ---- setup (a): the lane's map entries, scales and zero points
  const rsrc_t rf = make_rsrc(fmap, (uint32_t)(NM * (int64_t)H * 4));
  const rsrc_t rs = make_rsrc(scale, (uint32_t)(NP * (int64_t)H * 4));
  const rsrc_t rz = make_rsrc(zp, (uint32_t)(NP * (int64_t)H));
  const uint32_t lo4 = active ? (uint32_t)h0 * 4u : kOOB;
  const uint32_t lo1 = active ? (uint32_t)h0 : kOOB;
  v4u fv[NM][2];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    fv[m][0] = __builtin_amdgcn_raw_buffer_load_b128(rf, lo4, (uint32_t)(m * H * 4), 0);
    fv[m][1] = __builtin_amdgcn_raw_buffer_load_b128(rf, lo4 + 16u, (uint32_t)(m * H * 4), 0);
  }
  v4u sv[NP][2];
  v2u zv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    sv[p][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, lo4, (uint32_t)(p * H * 4), 0);
    sv[p][1] = __builtin_amdgcn_raw_buffer_load_b128(rs, lo4 + 16u, (uint32_t)(p * H * 4), 0);
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(rz, lo1, (uint32_t)(p * H), 0);
    zv[p] = v2u{t[0], t[1]};
  }
  issue_fence();

  // ---- the tile's geometry per map, from the map entries of its first
  // feature and of the next tile's (scalar loads): the slot of its first
  // int4 feature, and the run [ilo, ilo + nb) of BF16 indices inside it. A
  // feature h with slot j has h - j BF16 features below it; a BF16 feature
  // with index i has i. So the ring's loads need nothing from the lanes'
  // setup and go out right behind it.
  uint32_t abase[NM];   // dword where the code span of a row starts
  int ilo[NP], nbp[NP], off[NP + 1];
  const bool last_tile = f0 + kWinTile >= H;
  // Every map's two reads are issued together, from an index that is always
  // in range (on the last tile the second is not used), and pinned in scalar
  // registers before any is used: otherwise the compiler moves each read
  // under the condition that uses it, with a wait of its own, and the maps'
  // reads follow one another (eight round trips for per-shard sets).
  const int fnext = last_tile ? f0 : f0 + kWinTile;
  int fa[NM], fb[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int32_t* fr = fmap + (kPs ? (int64_t)m * H : 0);
    fa[m] = fr[f0];
    fb[m] = fr[fnext];
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    settle_s(fa[m]);
    settle_s(fb[m]);
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int ia = fa[m] >= 0 ? f0 - fa[m] : -1 - fa[m];
    const int ib = last_tile ? k : (fb[m] >= 0 ? f0 + kWinTile - fb[m] : -1 - fb[m]);
    ilo[m] = ia;
    nbp[m] = ib - ia;
    // the lanes' 8-byte windows start at or after the first int4 slot's
    // 4-byte aligned byte, or at pitch - 8 when pulled back inside the row
    const int cb0 = min(((f0 - ia) >> 1) & ~3, pitch - 8);
    abase[m] = ((uint32_t)cb0 >> 2) & ~1u;
  }
#pragma unroll
  for (int p = 1; p < NP; ++p) {
    if (!kPs) {
      ilo[p] = ilo[0];
      nbp[p] = nbp[0];
    }
  }
  off[0] = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) off[p + 1] = off[p] + nbp[p];
  const int E = off[NP];                           // entries per row
  const bool compact = E <= kOR * kWave;           // uniform

  // ---- the tile's code span per map. The lanes' windows are nondecreasing
  // in lane order and the last starts at most 63 dwords after the first, so
  // the span from the first window's dword (rounded down to even) holds at
  // most 66 dwords: the first 33 lanes load it with one coalesced 8-byte
  // load each, every code byte once. Each row's span goes through the
  // wave's LDS stage, where each lane reads its own window.
  uint32_t cl[NM];   // lane's load offset in the row
#pragma unroll
  for (int m = 0; m < NM; ++m)
    cl[m] = lane < kStageLanes ? 4u * abase[m] + 8u * (uint32_t)lane : kOOB;
  // BF16 entry e = off[p] + j of a row is index ilo[p] + j of shard p
  constexpr int kORA = kOR > 0 ? kOR : 1;   // array sizes (kOR = 0: no BF16 features)
  uint32_t e_off[kORA];
  int e_sp[kORA];   // the entry's shard
#pragma unroll
  for (int r = 0; r < kOR; ++r) {
    const int e = r * kWave + lane;
    int sp = 0, o = 0, lo = ilo[0];
#pragma unroll
    for (int p = 1; p < NP; ++p) {
      const bool ge = e >= off[p];
      sp = ge ? p : sp;
      o = ge ? off[p] : o;
      lo = ge ? ilo[p] : lo;
    }
    e_sp[r] = sp;
    e_off[r] = (compact && e < E)
                   ? (uint32_t)sp * (uint32_t)(T * k * 2) + (uint32_t)(lo + (e - o)) * 2u
                   : kOOB;
  }

  // ---- the ring: the first kR rows' code spans and BF16 entries. One
  // descriptor spans this wave's rows of every shard (the launcher keeps the
  // message under 2^31 bytes); the shard and row ride in the scalar offset.
  // A row past the wave's last loads through an empty descriptor (a scalar
  // choice). The code loads carry no streaming hint: the lines at tile
  // boundaries are read by two waves, and with the hint the L2 drops many
  // of them before the second read (about 20% more HBM reads, measured).
  const rsrc_t rpk = make_rsrc(packed + t0 * pitch,
                               (uint32_t)(((NP - 1) * T + nrows) * (int64_t)pitch));
  const rsrc_t rnone = make_rsrc(packed, 0u);
  const uint32_t shard_bytes = (uint32_t)(T * pitch);
  const rsrc_t ro = make_rsrc(outl + t0 * k, (uint32_t)(((NP - 1) * T + nrows) * (int64_t)k * 2));
  const rsrc_t rnone_o = make_rsrc(outl, 0u);
  // kAcc (a later group of shards): y holds the sum over the earlier groups,
  // and each row's values ride in the ring with its codes (a row past the
  // wave's last is out of this descriptor's range)
  const rsrc_t ryin = make_rsrc(static_cast<const char*>(y) + t0 * H * 4,
                                kAcc ? (uint32_t)((int64_t)nrows * H * 4) : 0u);
  const uint32_t yin_off = active ? (uint32_t)h0 * 4u : kOOB;
  v2u w[kR][NP];
  uint32_t ov[kR][kORA];
  float yp[kAcc ? kR : 1][kWinFeat];
  auto load_row = [&](int q, int row) {
    const bool ok = row < nrows;   // uniform
    const uint32_t so = (uint32_t)min(row, nrows - 1) * (uint32_t)pitch;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(ok ? rpk : rnone, cl[kPs ? p : 0],
                                                          so + (uint32_t)p * shard_bytes, 0);
      w[q][p] = v2u{t[0], t[1]};
    }
    const uint32_t soo = (uint32_t)(min(row, nrows - 1) * k * 2);
#pragma unroll
    for (int r = 0; r < kOR; ++r)
      ov[q][r] = __builtin_amdgcn_raw_buffer_load_b16(ok ? ro : rnone_o, e_off[r], soo, 0);
    if constexpr (kAcc) {
      const uint32_t soy = (uint32_t)row * (uint32_t)H * 4u;
      const v4u ya = __builtin_amdgcn_raw_buffer_load_b128(ryin, yin_off, soy, 0);
      const v4u yb = __builtin_amdgcn_raw_buffer_load_b128(ryin, yin_off + 16u, soy, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        yp[q][e] = __uint_as_float(ya[e]);
        yp[q][4 + e] = __uint_as_float(yb[e]);
      }
    }
  };
#pragma unroll
  for (int q = 0; q < kR; ++q) {
    load_row(q, q);
    issue_fence();
  }

  // ---- setup (b): per map, the code window and byte selectors.
  // A map entry f >= 0 is an int4 slot, f < 0 the BF16 index -1-f; inactive
  // lanes have neither. The lane's int4 features take consecutive slots from
  // the first one's,
  // jf, so feature e's nibble in the 8-byte window is n0 (jf's nibble) plus
  // the number of int4 features before e. The selectors therefore follow
  // from the lane's 8-bit int4 mask and n0; they are computed four features
  // at a time, one byte per feature: the mask's bits spread to bytes by one
  // multiplication, the ranks summed into bytes by another (no carries:
  // every byte stays below 23).
  uint32_t dwin[NM], selA[NM], selB[NM], mskA[NM], mskB[NM], bfm[NM];
  uint32_t i4A[NM], i4B[NM], hiA[NM], hiB[NM];   // per byte: int4 (1/0); high nibble (1/0)
  int bf1[NM];   // BF16 index of the lane's first BF16 feature (the others follow it)
  uint32_t i4any = 0;   // features int4 on some map
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    uint32_t qm = 0, jf = 0xFFFFFFFFu, jb = 0u;
#pragma unroll
    for (int e = 0; e < kWinFeat; ++e) {
      const uint32_t f = fv[m][e >> 2][e & 3];
      qm |= ((~f) >> 31) << e;
      // as unsigned, the BF16 entries (negative) are above every slot, and
      // the lowest BF16 index is the largest of them
      jf = min(jf, f);
      if (kPs) jb = max(jb, f);
    }
    qm = active ? qm : 0u;
    i4any |= qm;
    bfm[m] = active ? (~qm & 0xFFu) : 0u;
    bf1[m] = -1 - (int)jb;
    // 8 bytes at cb hold every code of the window; kept inside the row
    // (the launcher guarantees pitch >= 8)
    int base = qm ? (int)((jf >> 1) & ~3u) : 0;
    if (base + 8 > pitch) base -= 4;
    // the window's dword in the staged span (0 .. 64)
    dwin[m] = qm ? ((uint32_t)base >> 2) - abase[m] : 0u;
    const uint32_t n0 = jf - 2u * (uint32_t)base;   // 0..15 when the lane has an int4 feature
    const uint32_t sa = __umul24(qm & 0xFu, 0x204081u) & 0x01010101u;   // bit e -> byte e
    const uint32_t sb = __umul24(qm >> 4, 0x204081u) & 0x01010101u;
    // per byte: n0 plus the int4 features before it (exclusive prefix sums)
    const uint32_t na = __umul24(sa, 0x010100u) + (sa << 24) + splat_byte0(n0);
    const uint32_t nb = __umul24(sb, 0x010100u) + (sb << 24) +
                        splat_byte0(n0 + (uint32_t)__builtin_popcount(sa));
    // the code's byte (0x0C gives a zero byte) and nibble mask, zero where BF16
    auto sel4 = [](uint32_t i4, uint32_t n, uint32_t& sel, uint32_t& msk, uint32_t& hi) {
      const uint32_t keep = (i4 << 8) - i4;   // 0xFF where int4
      sel = ((n >> 1) & 0x7F7F7F7Fu & keep) | (0x0C0C0C0Cu & ~keep);
      const uint32_t odd = n & 0x01010101u;   // the code is a high nibble
      msk = (0x0F0F0F0Fu ^ ((odd << 8) - odd)) & keep;
      hi = odd & i4;
    };
    sel4(sa, na, selA[m], mskA[m], hiA[m]);
    sel4(sb, nb, selB[m], mskB[m], hiB[m]);
    i4A[m] = sa;
    i4B[m] = sb;
  }

  // ---- setup (c): the lanes' BF16 features (wave counts from ballots) and
  // the table row of each entry. Shared set: entry (p, i) -> row i - ilo.
  // One set per shard: through the inverse map that the owners write here.
  int any = 0;   // features BF16 on some shard
#pragma unroll
  for (int m = 0; m < NM; ++m) any |= (int)bfm[m];
  const int cnt_any = __builtin_popcount(any);
  const int pos0 = wave_prefix16(cnt_any, lane);   // table row of the lane's first
  const int nb_any = kPs ? wave_sum16(cnt_any) : nbp[0];
  const int umax = wave_max8(cnt_any);
  if constexpr (kPs) {
    if (compact) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        // the lane's BF16 features on shard p are its entries from `first` on,
        // in feature order. A short per-lane loop over just those features
        // (most lanes have none or one): all 8 features with dummy writes
        // cost 48 more instructions per shard.
        const int first = off[p] + bf1[p] - ilo[p];
        uint32_t rest = bfm[p];
#pragma unroll
        for (int rb = 0; rb < kWinFeat; ++rb) {
          if (rest == 0u) break;
          const int e = __builtin_ctz(rest);
          rest &= rest - 1u;
          inv[first + rb] = pos0 + __builtin_popcount((uint32_t)any & ((1u << e) - 1u));
        }
      }
    }
  }
  // zero the table rows of this tile (int4 shards of a BF16 feature stay 0)
  for (int i = lane; i < nb_any * NP && compact; i += kWave) tab[i] = 0.0f;
  wave_lds_sync();
  uint32_t e_dst[kORA];   // entry: LDS dword (past the entries: the lane's dummy)
#pragma unroll
  for (int r = 0; r < kOR; ++r) {
    const int e = r * kWave + lane;
    const bool live = compact && e < E;
    int row;
    if constexpr (kPs) {
      row = inv[live ? e : 0];
    } else {
      int o = 0;
#pragma unroll
      for (int p = 1; p < NP; ++p) o = e >= off[p] ? off[p] : o;
      row = e - o;
    }
    e_dst[r] = live ? (uint32_t)(row * NP + e_sp[r]) : (uint32_t)(dummy - tab) + lane;
  }
  wave_lds_sync();

  // ---- per-lane constants (their loads are older than the ring). Per map
  // and feature: int4 or not, and the factor its scale carries (1/16 for a
  // high nibble). A term of a shard where the feature is BF16 has code 0 and
  // scale 0: with one set its products, even non-finite ones, stay in the
  // feature's own accumulator, which its BF16 sum replaces; per-shard sets
  // select scale 0 so that such a shard adds exactly 0 to the int4 part.
  // One set: the scales are held multiplied by 2^24 (fma_h0/fma_h1). A
  // scale of 2^104 or more would overflow there: a wave with such a lane
  // (`huge`, never in practice) recomputes all its outputs term by term
  // after the row loop. Per-shard sets, whose kernels have no registers to
  // spare, convert each code and use fmaf.
  constexpr bool kMix = !kPs;
  constexpr float kMs = kMix ? kTwo24 : 1.0f;
  float sc[NP][kWinFeat], bias[kWinFeat];
  // the scale's factor: kMs (low nibble), kMs/16 (high nibble), 0 (BF16 on the map)
  float mh[NM][kWinFeat];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int e = 0; e < kWinFeat; ++e) {
      const int sh = 8 * (e & 3);
      const float is4 = (float)(((e < 4 ? i4A[m] : i4B[m]) >> sh) & 0xFFu);
      const float ishi = (float)(((e < 4 ? hiA[m] : hiB[m]) >> sh) & 0xFFu);
      mh[m][e] = fmaf(-0.9375f, ishi, is4) * kMs;   // exact
    }
  }
#pragma unroll
  for (int e = 0; e < kWinFeat; ++e) bias[e] = 0.0f;
  bool over = false;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int m = kPs ? p : 0;
#pragma unroll
    for (int e = 0; e < kWinFeat; ++e) {
      const float s = __uint_as_float(sv[p][e >> 2][e & 3]);
      const float z = (float)((zv[p][e >> 2] >> (8 * (e & 3))) & 0xFFu);
      // -sum_p z*s over the int4 shards, in shard order from +0. With one
      // set, a BF16 feature's constant is never used (its sum replaces it).
      const float b = fmaf(-z, s, bias[e]);
      const bool q4 = mh[m][e] != 0.0f;
      bias[e] = (kPs && !q4) ? bias[e] : b;
      sc[p][e] = kPs ? (q4 ? s * mh[m][e] : 0.0f) : s * mh[m][e];
      // (+-inf: the scale times 2^24 overflowed; a NaN scale too)
      if (kMix) over |= !(fabsf(sc[p][e]) <= 3.0e38f);
      settle(sc[p][e]);
    }
  }
#pragma unroll
  for (int e = 0; e < kWinFeat; ++e) settle(bias[e]);
  const bool huge = __ballot(over) != 0ull;   // uniform
  // features the post-loop pass recomputes: every active one when huge,
  // else the BF16 ones of a tile past its entry registers
  const int redo = huge ? (active ? 0xFF : 0) : (compact ? 0 : any);
  // y stores. bf16: the lane's 8 values are 16 contiguous bytes, so one
  // store covers the wave's 1 KB. fp32: the lane's 32 bytes go through the
  // wave's LDS row (values 0-3 of every lane in the first half, 4-7 in the
  // second), and lane m stores features 4m..4m+3 and 256+4m..256+4m+3 of
  // the tile: each store instruction writes 1 KB of whole lines.
  const int e_first = __builtin_ctz(any | (1 << kWinFeat));   // kWinFeat: none
  const int any_rest = any & (any - 1);                      // BF16 features past the first
  // The owner's BF16 sum into its feature eu: one set per shard adds it to
  // the int4 part; with one set it is the whole value (the int4 part is +0).
  // A select, so no other feature ever sees the sum.
  // Features BF16 on every map (with one set: every BF16 feature). In a
  // later group of shards their owner sum starts from the earlier groups' y
  // and replaces the value, so a feature BF16 on every shard keeps its sum
  // in shard order from +0 across groups; a feature with int4 terms in the
  // group adds its BF16 sum to them.
  const int allbf = kPs ? (any & ~(int)i4any) : any;
  auto place = [&](float (&acc)[kWinFeat], int eu, float o) {
#pragma unroll
    for (int e = 0; e < kWinFeat; ++e) {
      const bool repl = !kPs || (kAcc && ((allbf >> e) & 1));
      acc[e] = (e == eu) ? (repl ? o : __fadd_rn(acc[e], o)) : acc[e];
    }
  };
  const uint32_t st_off = active ? (uint32_t)h0 * kYB : kOOB;
  const uint32_t st_a = (f0 + 4 * lane < H) ? (uint32_t)(f0 + 4 * lane) * 4u : kOOB;
  const uint32_t st_b = (f0 + 256 + 4 * lane < H) ? (uint32_t)(f0 + 256 + 4 * lane) * 4u : kOOB;
  const uint32_t ld_a = (uint32_t)((lane & 1) * 256 + (lane >> 1) * 4);          // dwords
  const uint32_t ld_b = (uint32_t)((lane & 1) * 256 + (32 + (lane >> 1)) * 4);
  char* const ybase = static_cast<char*>(y) + t0 * H * (int64_t)kYB;
  // (a row past the wave's last stores through an empty descriptor; the
  // stores take an immediate zero scalar offset: a store wider than 64 bits
  // reads its data after issue, and only with an immediate scalar offset
  // does the compiler keep the next instruction from overwriting them)
  const uint32_t ybytes_row = (uint32_t)H * kYB;
  // wave-uniform switches of the row loop, held in scalar registers
  const bool do_tab = __builtin_amdgcn_readfirstlane((int)(compact && nb_any > 0)) != 0;
  const bool do_own = __builtin_amdgcn_readfirstlane((int)(compact && umax > 0)) != 0;
  char* yrow_ptr = ybase;   // advanced by one row per row (uniform)

  int base = 0;
  do {
#pragma unroll
    for (int q = 0; q < kR; ++q) {
      const int row = base + q;
      // the row's code spans and BF16 entries into LDS; then each lane's
      // code windows and the owners' first table row
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        uint32_t* const dst = stage + 2 * lane * kSP + 2 * p;
        dst[0] = w[q][p][0];
        dst[kSP] = w[q][p][1];
      }
      if (do_tab) {
#pragma unroll
        for (int r = 0; r < kOR; ++r) tab[e_dst[r]] = __uint_as_float(ov[q][r] << 16);
      }
      wave_lds_sync();
      v2u x[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t* src = stage + dwin[kPs ? p : 0] * kSP + 2 * p;
        x[p] = v2u{src[0], src[kSP]};
      }
      // the owner's first BF16 feature: its row summed in shard order from +0
      // (a later group of shards: from the earlier groups' sum)
      float o = 0.0f;
      if (do_own) {
        if constexpr (kAcc) o = ((allbf >> e_first) & 1) ? pick8(yp[q], e_first) : 0.0f;
        const float* t = tab + (cnt_any > 0 ? pos0 : 0) * NP;
        if constexpr (NP % 4 == 0) {
#pragma unroll
          for (int p = 0; p < NP; p += 4) {
            const v4f f = *reinterpret_cast<const v4f*>(t + p);
            o = __fadd_rn(__fadd_rn(__fadd_rn(__fadd_rn(o, f[0]), f[1]), f[2]), f[3]);
          }
        } else {
#pragma unroll
          for (int p = 0; p < NP; ++p) o = __fadd_rn(o, t[p]);
        }
      }
      issue_fence();   // the read goes out before the arithmetic below
      float acc[kWinFeat];
#pragma unroll
      for (int e = 0; e < kWinFeat; ++e) acc[e] = kAcc ? __fadd_rn(yp[q][e], bias[e]) : bias[e];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int m = kPs ? p : 0;
        uint32_t a = __builtin_amdgcn_perm(x[p][1], x[p][0], selA[m]) & mskA[m];
        uint32_t b = __builtin_amdgcn_perm(x[p][1], x[p][0], selB[m]) & mskB[m];
        if constexpr (!kMix) {
          // kept whole: each byte converts with one v_cvt_f32_ubyteN
          opaque(a);
          opaque(b);
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            acc[bb] = fmaf((float)((a >> (8 * bb)) & 0xFFu), sc[p][bb], acc[bb]);
            acc[4 + bb] = fmaf((float)((b >> (8 * bb)) & 0xFFu), sc[p][4 + bb], acc[4 + bb]);
          }
          continue;
        }
        // one code byte per 16-bit half: f16 denormals
        const uint32_t a01 = __builtin_amdgcn_perm(0u, a, kSpread01);
        const uint32_t a23 = __builtin_amdgcn_perm(0u, a, kSpread23);
        const uint32_t b01 = __builtin_amdgcn_perm(0u, b, kSpread01);
        const uint32_t b23 = __builtin_amdgcn_perm(0u, b, kSpread23);
        acc[0] = fma_h0(a01, sc[p][0], acc[0]);
        acc[1] = fma_h1(a01, sc[p][1], acc[1]);
        acc[2] = fma_h0(a23, sc[p][2], acc[2]);
        acc[3] = fma_h1(a23, sc[p][3], acc[3]);
        acc[4] = fma_h0(b01, sc[p][4], acc[4]);
        acc[5] = fma_h1(b01, sc[p][5], acc[5]);
        acc[6] = fma_h0(b23, sc[p][6], acc[6]);
        acc[7] = fma_h1(b23, sc[p][7], acc[7]);
      }
      // (kAcc: the owners' later features still need this row's y after the
      // refill below reloads its slot)
      float yq[kAcc ? kWinFeat : 1];
      if constexpr (kAcc) {
#pragma unroll
        for (int e = 0; e < kWinFeat; ++e) yq[e] = yp[q][e];
      }
      // this row's registers are consumed: refill the slot kR rows ahead
      load_row(q, row + kR);
      issue_fence();
      if (do_own) {
        place(acc, e_first, o);
        int rest = any_rest;
        for (int u = 1; u < umax; ++u) {   // lanes with several BF16 features
          const float* t = tab + (u < cnt_any ? pos0 + u : 0) * NP;
          const int eu = rest ? __builtin_ctz(rest) : kWinFeat;
          float ou = 0.0f;
          if constexpr (kAcc) ou = ((allbf >> eu) & 1) ? pick8(yq, eu) : 0.0f;
#pragma unroll
          for (int p = 0; p < NP; ++p) ou = __fadd_rn(ou, t[p]);
          place(acc, eu, ou);
          rest &= rest - 1;
        }
      }
      if constexpr (kAcc) {
        // the post-loop pass continues these features from what the earlier
        // groups summed, so the loop stores that unchanged
        if (redo) {
#pragma unroll
          for (int e = 0; e < kWinFeat; ++e) acc[e] = ((redo >> e) & 1) ? yq[e] : acc[e];
        }
      }
      // (a row past the wave's last: no records, every store dropped)
      const rsrc_t ry = make_rsrc(yrow_ptr, row < nrows ? ybytes_row : 0u);
      yrow_ptr += ybytes_row;
      if constexpr (kBf) {
        __builtin_amdgcn_raw_buffer_store_b128(
            v4u{bf16_pair(acc[0], acc[1]), bf16_pair(acc[2], acc[3]), bf16_pair(acc[4], acc[5]),
                bf16_pair(acc[6], acc[7])},
            ry, st_off, 0, kStream);
      } else {
        *reinterpret_cast<v4f*>(yrow + 4 * lane) = v4f{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<v4f*>(yrow + 256 + 4 * lane) = v4f{acc[4], acc[5], acc[6], acc[7]};
        wave_lds_sync();
        const v4f ya = *reinterpret_cast<const v4f*>(yrow + ld_a);
        const v4f yb = *reinterpret_cast<const v4f*>(yrow + ld_b);
        __builtin_amdgcn_raw_buffer_store_b128(
            v4u{__float_as_uint(ya[0]), __float_as_uint(ya[1]), __float_as_uint(ya[2]),
                __float_as_uint(ya[3])},
            ry, st_a, 0, kStream);
        __builtin_amdgcn_raw_buffer_store_b128(
            v4u{__float_as_uint(yb[0]), __float_as_uint(yb[1]), __float_as_uint(yb[2]),
                __float_as_uint(yb[3])},
            ry, st_b, 0, kStream);
      }
      wave_lds_sync();   // the next row overwrites the stage, the table and the LDS row
    }
    base += kR;
  } while (base < nrows);

  if (!compact || huge) {   // uniform
    // More BF16 entries than the registers hold: the loop stored only the
    // int4 part of these features (or, when huge, nothing valid). Once those
    // stores are complete, each owner recomputes these features term by
    // term (fl(q - z) * s or the BF16 value, in shard order from +0) and
    // stores the sums. The maps and parameters are read again here, so the
    // loop does not keep them live.
    __builtin_amdgcn_s_waitcnt(0);
    int rest = redo;
    while (rest) {
      const int e = __builtin_ctz(rest);
      rest &= rest - 1;
      const int64_t h = h0 + e;
      for (int r = 0; r < nrows; ++r) {
        char* d = ybase + ((int64_t)r * H + h) * kYB;
        float o = kAcc ? *reinterpret_cast<const float*>(d) : 0.0f;
        for (int p = 0; p < NP; ++p) {
          const int f = fmap[(kPs ? (int64_t)p * H : 0) + h];
          const int64_t rowg = (int64_t)p * T + t0 + r;
          float term;
          if (f >= 0) {
            const uint32_t byte = packed[rowg * pitch + (f >> 1)];
            const float qv = (float)((f & 1) ? (byte >> 4) : (byte & 0xFu));
            term = __fmul_rn(__fsub_rn(qv, (float)zp[p * H + h]), scale[p * H + h]);
          } else {
            term = bf16_to_f32(outl[rowg * k + (-1 - f)]);
          }
          o = __fadd_rn(o, term);
        }
        if constexpr (kBf)
          *reinterpret_cast<uint16_t*>(d) = bf16_rne(o);
        else
          *reinterpret_cast<float*>(d) = o;
      }
    }
  }
}

template <bool kPs, bool kBf>
__global__ __launch_bounds__(256) void dq_general_kernel(
    const uint8_t* __restrict__ packed, int64_t pitch, const uint16_t* __restrict__ outl, int64_t P,
    int64_t T, int64_t H, int64_t k, const float* __restrict__ scale,
    const uint8_t* __restrict__ zp, const int32_t* __restrict__ fmap, void* __restrict__ y) {
  const int64_t n = T * H;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t t = i / H, h = i % H;
    float acc = 0.0f;
    for (int64_t p = 0; p < P; ++p) {
      const int64_t f = fmap[(kPs ? p * H : 0) + h];
      const int64_t row = p * T + t;
      float term;
      if (f >= 0) {
        const uint32_t byte = packed[row * pitch + (f >> 1)];
        const float q = (float)((f & 1) ? (byte >> 4) : (byte & 0xFu));
        term = __fmul_rn(__fsub_rn(q, (float)zp[p * H + h]), scale[p * H + h]);   // q - z exact
      } else {
        term = bf16_to_f32(outl[row * k + (-1 - f)]);
      }
      acc = __fadd_rn(acc, term);
    }
    if constexpr (kBf)
      static_cast<uint16_t*>(y)[i] = bf16_rne(acc);
    else
      static_cast<float*>(y)[i] = acc;
  }
}

template <int NP, int kOR, int kR, bool kPs, bool kBf, bool kAcc>
static void launch_window(const uint8_t* packed, int64_t pitch, const uint16_t* outl, int64_t T,
                          int64_t H, int64_t k, int ntiles, int rpw, int64_t nrowblk,
                          const float* scale, const uint8_t* zp, const int32_t* fmap, void* y,
                          hipStream_t s) {
  const int64_t ntgrp = (ntiles + kDqWaves - 1) / kDqWaves;
  const size_t lds = (size_t)kDqWaves * win_lds_dwords<NP, kOR, kPs, kBf>() * 4;
  dq_window_kernel<NP, kOR, kR, kPs, kBf, kAcc><<<(unsigned)xcd_grid(ntgrp, nrowblk), 256, lds, s>>>(
      packed, (int)pitch, outl, T, (int)H, (int)k, ntiles, rpw, nrowblk, scale, zp, fmap, y);
}

// Shards per group for per-shard sets: their kernels hold every shard's
// selectors and scales in registers, and past 6 shards the earlier groups' y
// no longer fits beside them.
constexpr int kPsGroup = 6;

template <bool kPs, bool kBf, bool kAcc>
static void dispatch_window(int64_t P, int kor, const uint8_t* packed, int64_t pitch,
                            const uint16_t* outl, int64_t T, int64_t H, int64_t k, int ntiles,
                            int rpw, int64_t nrowblk, const float* scale, const uint8_t* zp,
                            const int32_t* fmap, void* y, hipStream_t s) {
#define BTQ_WIN_ARGS packed, pitch, outl, T, H, k, ntiles, rpw, nrowblk, scale, zp, fmap, y, s
#define BTQ_WIN_CASE(n)                                                         \
  case n:                                                                       \
    if constexpr (kPs && kAcc && n > kPsGroup) {                                \
      /* never launched: per-shard groups hold at most kPsGroup shards */       \
    } else if (kor == 4) {                                                      \
      launch_window<n, 4, kDqRing, kPs, kBf, kAcc>(BTQ_WIN_ARGS);               \
    } else if constexpr (kPs || kAcc) {                                         \
      launch_window<n, 2, kDqRing, kPs, kBf, kAcc>(BTQ_WIN_ARGS);               \
    } else {                                                                    \
      if (kor == 2)                                                             \
        launch_window<n, 2, kDqRing, kPs, kBf, kAcc>(BTQ_WIN_ARGS);             \
      else                                                                      \
        launch_window<n, 0, kDqRing, kPs, kBf, kAcc>(BTQ_WIN_ARGS);             \
    }                                                                           \
    break;
  switch (P) {
    BTQ_WIN_CASE(1)
    BTQ_WIN_CASE(2)
    BTQ_WIN_CASE(3)
    BTQ_WIN_CASE(4)
    BTQ_WIN_CASE(5)
    BTQ_WIN_CASE(6)
    BTQ_WIN_CASE(7)
    BTQ_WIN_CASE(8)
  }
#undef BTQ_WIN_CASE
#undef BTQ_WIN_ARGS
}

template <bool kPs, bool kBf>
static hipError_t launch_decompress_t(const uint8_t* packed, int64_t pitch, const uint16_t* outl,
                                      int64_t P, int64_t T, int64_t H, int64_t k,
                                      const float* scale, const uint8_t* zp, const int32_t* fmap,
                                      void* y, hipStream_t s) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t nm = kPs ? P : 1;
  // Window kernel: whole 8-feature lane windows; the code window of 8 bytes
  // inside every row (pitch >= 8, dword-aligned rows); 16-byte aligned
  // per-feature arrays and y; each descriptor under 2^31 bytes (the
  // parameter arrays, and the message and outlier block of up to 8 shards).
  const bool shape_ok = H % 8 == 0 && pitch >= 8 && pitch % 4 == 0 &&
                        (uintptr_t)packed % 4 == 0 && (uintptr_t)fmap % 16 == 0 &&
                        (uintptr_t)scale % 16 == 0 && (uintptr_t)zp % 8 == 0 &&
                        (uintptr_t)y % 16 == 0 && (uintptr_t)outl % 2 == 0 &&
                        nm * H * 4 < lim && 64 * H * 4 < lim;
  auto group_ok = [&](int64_t np) {
    return np * H * 4 < lim && np * T * k * 2 < lim && np * T * pitch < lim;
  };
  const int ntiles = (int)((H + kWinTile - 1) / kWinTile);
  int64_t rpw64 = (ntiles * T + kDqWavesTwo - 1) / kDqWavesTwo;
  if (rpw64 < dq_min_rows_two(kPs, kBf)) rpw64 = (ntiles * T + kDqWavesOne - 1) / kDqWavesOne;
  rpw64 = (rpw64 + kDqRing - 1) / kDqRing * kDqRing;
  if (rpw64 < kDqRing) rpw64 = kDqRing;
  if (rpw64 > 64) rpw64 = 64;
  const int rpw = (int)rpw64;
  const int64_t nrowblk = (T + rpw - 1) / rpw;
  // BF16 entry registers per row: none without BF16 features (one set); 2
  // (128 entries per tile-row) while the tiles hold at most 64 on average;
  // else 4
  auto entry_regs = [&](int64_t np) {
    return k == 0 ? 0 : (np * k > int64_t(kWave) * ntiles ? 4 : 2);
  };
  // shards per launch: at most 8, and few enough that a group's message and
  // outlier block stay under 2^31 bytes
  int64_t gs = 8;
  while (gs > 0 && !group_ok(gs)) --gs;
  if (P <= gs && shape_ok) {
    dispatch_window<kPs, kBf, false>(P, entry_regs(P), packed, pitch, outl, T, H, k, ntiles, rpw,
                                     nrowblk, scale, zp, fmap, y, s);
    return hipGetLastError();
  }
  if constexpr (!kBf) {
    // More shards than one launch takes (more than 8, or a message past 2^31
    // bytes; fp32 output): one launch per group of shards, in shard order
    // (gs shards, or at most kPsGroup with per-shard sets). The first writes
    // y; each later one starts every feature from y, so a feature BF16 on
    // every shard keeps its sum in shard order from +0 across the groups.
    const int64_t gg = kPs ? (gs < kPsGroup ? gs : kPsGroup) : gs;
    if (P > gs && gg >= 1 && shape_ok) {
      for (int64_t g0 = 0; g0 < P; g0 += gg) {
        const int64_t np = P - g0 < gg ? P - g0 : gg;
        const int kor = kPs ? (np * k > int64_t(kWave) * ntiles ? 4 : 2) : entry_regs(np);
        const uint8_t* pk_g = packed + g0 * T * pitch;
        const uint16_t* ol_g = outl + g0 * T * k;
        const int32_t* fm_g = kPs ? fmap + g0 * H : fmap;
        if (g0 == 0)
          dispatch_window<kPs, false, false>(np, kor, pk_g, pitch, ol_g, T, H, k, ntiles, rpw,
                                             nrowblk, scale, zp, fm_g, y, s);
        else
          dispatch_window<kPs, false, true>(np, kor, pk_g, pitch, ol_g, T, H, k, ntiles, rpw,
                                            nrowblk, scale + g0 * H, zp + g0 * H, fm_g, y, s);
      }
      return hipGetLastError();
    }
  }
  int64_t blocks = (T * H + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  dq_general_kernel<kPs, kBf><<<(unsigned)blocks, 256, 0, s>>>(packed, pitch, outl, P, T, H, k,
                                                               scale, zp, fmap, y);
  return hipGetLastError();
}

hipError_t launch_decompress(const uint8_t* packed, int64_t pitch, const uint16_t* outl, int64_t P,
                             int64_t T, int64_t H, int64_t k, const float* scale,
                             const uint8_t* zp, const int32_t* fmap, bool per_shard, void* y,
                             bool bf16, hipStream_t s) {
  if (per_shard)
    return bf16 ? launch_decompress_t<true, true>(packed, pitch, outl, P, T, H, k, scale, zp, fmap,
                                                  y, s)
                : launch_decompress_t<true, false>(packed, pitch, outl, P, T, H, k, scale, zp,
                                                   fmap, y, s);
  return bf16 ? launch_decompress_t<false, true>(packed, pitch, outl, P, T, H, k, scale, zp, fmap,
                                                 y, s)
              : launch_decompress_t<false, false>(packed, pitch, outl, P, T, H, k, scale, zp, fmap,
                                                  y, s);
}

}  // namespace btq
