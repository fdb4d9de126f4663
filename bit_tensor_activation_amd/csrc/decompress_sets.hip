// Receiver for per-shard BF16 sets: every shard keeps its own k features in
// BF16, so a feature's int4 slot differs from shard to shard and the receiver
// looks each one up in that shard's map.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm": Inference
// bullet (convert every device's tensor back and sum across devices). One set
// per shard is a reading of the Selection bullet, whose ranges are per
// device.
//
// y[t,h] = sum over p = 0, 1, ... of term_p, in fp32 from +0, where term_p is
// fl(q - z) * s with shard p's code q of feature h at slot fmap[p,h], or the
// exact BF16 value outliers[p,t,-1-fmap[p,h]].
#include "common.hpp"

namespace btq {

constexpr int kSetRows = 4;   // token rows per thread
constexpr int kSetFeat = 8;   // consecutive features per thread
constexpr int kSetBlockFeat = 256 * kSetFeat;

// Thread: features [h0, h0+8) of kSetRows token rows; a block covers 2048
// features. Per shard, in shard order, the thread reads the shard's map,
// scales and zero points of its 8 features (small tables that stay in L2),
// then the codes of every row. The int4 features among the 8 take
// consecutive slots of shard p starting at the first one's slot jf, so the
// two aligned dwords at byte (jf/2) & ~3 hold all their nibbles. The
// shard's BF16 features come from its outlier block.
__global__ __launch_bounds__(256) void decompress_sets_kernel(
    const uint8_t* __restrict__ packed, int pitch, const uint16_t* __restrict__ outl, int64_t P,
    int64_t T, int H, int k, const float* __restrict__ scale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ fmap, float* __restrict__ y, int nfblk) {
  const int64_t b = blockIdx.x;
  const int fb = (int)(b % nfblk);
  const int64_t rb = b / nfblk;
  const int h0 = fb * kSetBlockFeat + (int)threadIdx.x * kSetFeat;
  if (h0 >= H) return;   // no block barrier below
  const int64_t t0 = rb * kSetRows;
  const int nrows = (int)min((int64_t)kSetRows, T - t0);

  float acc[kSetRows][kSetFeat];
#pragma unroll
  for (int r = 0; r < kSetRows; ++r)
#pragma unroll
    for (int e = 0; e < kSetFeat; ++e) acc[r][e] = 0.0f;

  for (int64_t p = 0; p < P; ++p) {
    const int64_t ph = p * H + h0;
    const int4 fa = *reinterpret_cast<const int4*>(fmap + ph);
    const int4 fc = *reinterpret_cast<const int4*>(fmap + ph + 4);
    const float4 sa = *reinterpret_cast<const float4*>(scale + ph);
    const float4 sc = *reinterpret_cast<const float4*>(scale + ph + 4);
    const uint2 zz = *reinterpret_cast<const uint2*>(zp + ph);
    const int f[kSetFeat] = {fa.x, fa.y, fa.z, fa.w, fc.x, fc.y, fc.z, fc.w};
    const float s[kSetFeat] = {sa.x, sa.y, sa.z, sa.w, sc.x, sc.y, sc.z, sc.w};
    int zi[kSetFeat];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zi[e] = (int)((zz.x >> (8 * e)) & 0xFFu);
      zi[e + 4] = (int)((zz.y >> (8 * e)) & 0xFFu);
    }
    int jf = 0x7FFFFFFF;   // first int4 slot among the 8 features
    bool any_bf16 = false;
#pragma unroll
    for (int e = 0; e < kSetFeat; ++e) {
      if (f[e] >= 0) jf = min(jf, f[e]);
      any_bf16 |= f[e] < 0;
    }
    const bool any_int4 = jf != 0x7FFFFFFF;
    // as in the register kernel: the 8-byte window never passes the row's end
    uint32_t base = any_int4 ? (((uint32_t)jf >> 1) & ~3u) : 0u;
    if (base + 8u > (uint32_t)pitch) base -= 4u;
    const int64_t row0 = p * T + t0;
    // Rows past nrows and threads with no int4 feature read out of range
    // (zeros, no traffic). A dword past the end of the last row is out of
    // range too; one past the end of an earlier row reads the next row's
    // bytes, whose nibbles are never used.
    const rsrc_t rp = make_rsrc(packed + row0 * pitch, (uint32_t)nrows * (uint32_t)pitch);
    uint32_t w0[kSetRows], w1[kSetRows];
#pragma unroll
    for (int r = 0; r < kSetRows; ++r) {
      const uint32_t o = (r < nrows && any_int4) ? base + (uint32_t)r * (uint32_t)pitch : kOOB;
      w0[r] = __builtin_amdgcn_raw_buffer_load_b32(rp, o, 0, kStream);
      w1[r] = __builtin_amdgcn_raw_buffer_load_b32(rp, o + 4u, 0, kStream);
    }
    uint32_t ob[kSetRows][kSetFeat];
#pragma unroll
    for (int r = 0; r < kSetRows; ++r)
#pragma unroll
      for (int e = 0; e < kSetFeat; ++e) ob[r][e] = 0u;
    if (any_bf16) {
#pragma unroll
      for (int r = 0; r < kSetRows; ++r) {
        if (r >= nrows) break;
#pragma unroll
        for (int e = 0; e < kSetFeat; ++e)
          if (f[e] < 0) ob[r][e] = outl[(row0 + r) * k + (-1 - f[e])];
      }
    }
#pragma unroll
    for (int r = 0; r < kSetRows; ++r) {
      const uint64_t wv = (uint64_t)w0[r] | ((uint64_t)w1[r] << 32);
#pragma unroll
      for (int e = 0; e < kSetFeat; ++e) {
        // slot f[e] sits at nibble f[e] - 2*base (0..15) of the 16 loaded
        const uint32_t q = (uint32_t)(wv >> (4 * ((f[e] - (int)(2 * base)) & 15))) & 15u;
        const float dq = __fmul_rn((float)((int)q - zi[e]), s[e]);
        const float term = f[e] >= 0 ? dq : bf16_to_f32(ob[r][e]);
        acc[r][e] = __fadd_rn(acc[r][e], term);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kSetRows; ++r) {
    if (r >= nrows) break;
    float* d = y + (t0 + r) * H + h0;
    *reinterpret_cast<float4*>(d) = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
  }
}

// Register kernel (P <= 8). A wave owns a window of 256 features (4 per
// lane) over rows_per_wave token rows; a block, 4 adjacent windows. Before
// the rows, it reduces every shard's map, zero points and scales of its 4
// features to 8 registers per shard:
//   * nib: the bit shift of each int4 feature's code within the 64 bits
//     loaded at byte `pb` of the row (the lane's int4 features take
//     consecutive slots of the shard, so two aligned dwords hold them);
//   * zm: the 4 zero points (4 bits each) and the int4/BF16 mask;
//   * orl: the position of each BF16 feature inside the window's run of the
//     shard's outlier block (a shard's BF16 features are listed in ascending
//     h, so the window's ones are a contiguous run [ilo, ihi));
//   * the 4 scales.
// Per row, it issues the two code dwords and one coalesced load of the run
// for all shards at once (lane l holds run element ilo + l; RO registers for
// runs longer than 64). Two register sets take turns, so the next row's
// loads are in flight during a row's arithmetic. Each lane fetches its BF16
// values from the holding lanes with ds_bpermute, or, for runs longer than
// 64, from a per-row LDS copy of the run. Terms are summed in shard order
// from +0.
template <int NP, int RO>
__global__ __launch_bounds__(256) void decompress_sets_reg_kernel(
    const uint8_t* __restrict__ packed, int pitch, const uint16_t* __restrict__ outl, int64_t T,
    int H, int k, const float* __restrict__ scale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ fmap, float* __restrict__ y, int nwin, int nwg,
    int rows_per_wave, int64_t nrb) {
  // unit = block of token rows; its nwg blocks (4 windows each) run on one
  // XCD, so the cache lines that neighbouring windows share are fetched into
  // one L2 once
  int64_t rb, sub;
  if (!xcd_unit_block(blockIdx.x, nwg, nrb, &rb, &sub)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = (int)sub * 4 + wave;
  if (c >= nwin) return;   // no block barrier below
  const int hw0 = c * 256;
  const int h0 = hw0 + 4 * lane;
  const bool active = h0 < H;   // lanes past H still take part in the bpermutes
  const int hh = active ? h0 : hw0;
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min((int64_t)rows_per_wave, T - t0);
  const int hend = min(hw0 + 256, H);

  uint32_t nib[NP], zm[NP], orl[NP], pb[NP], olx[NP][RO];
  float sc[NP][4];
  // One descriptor per tensor (the launcher keeps both below 2^30 bytes);
  // a shard's row offset is part of the lane offsets.
  const int64_t nrows_total = NP * T;
  const rsrc_t rp = make_rsrc(packed, (uint32_t)(nrows_total * pitch));
  const rsrc_t ro = make_rsrc(outl, (uint32_t)(nrows_total * k * 2));
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t ph = (int64_t)p * H + hh;
    const int4 fv = *reinterpret_cast<const int4*>(fmap + ph);
    const float4 sv = *reinterpret_cast<const float4*>(scale + ph);
    const uint32_t zv = *reinterpret_cast<const uint32_t*>(zp + ph);
    const int f[4] = {fv.x, fv.y, fv.z, fv.w};
    sc[p][0] = sv.x;
    sc[p][1] = sv.y;
    sc[p][2] = sv.z;
    sc[p][3] = sv.w;
    // the window's run of shard p's BF16 features: BF16 features below h are
    // h - fmap[h] when h is int4, -1 - fmap[h] when it is BF16, k at h = H
    const int f0 = __builtin_amdgcn_readfirstlane(f[0]);   // lane 0 holds h = hw0
    const int ilo = f0 >= 0 ? hw0 - f0 : -1 - f0;
    int ihi = k;
    if (hend < H) {
      const int g = fmap[(int64_t)p * H + hend];
      ihi = g >= 0 ? hend - g : -1 - g;
    }
    const int nrun = ihi - ilo;
    int jf = 0x7FFFFFFF;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (f[e] >= 0) jf = min(jf, f[e]);
    const bool any_int4 = jf != 0x7FFFFFFF;
    // 8 bytes from the dword holding slot jf; moved back one dword where that
    // would pass the row's end (the codes end within the row, so the window
    // still holds them, at nibbles up to 15)
    uint32_t base = any_int4 ? (((uint32_t)jf >> 1) & ~3u) : 0u;
    if (base + 8u > (uint32_t)pitch) base -= 4u;
    uint32_t n = 0, z = 0, o = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool i4 = f[e] >= 0;
      const uint32_t sh = i4 ? 4u * (uint32_t)(f[e] - (int)(2 * base)) : 0u;   // <= 60
      const uint32_t rel = i4 ? 0u : (uint32_t)(-1 - f[e] - ilo);              // < 256
      n |= sh << (8 * e);
      o |= rel << (8 * e);
      z |= (((zv >> (8 * e)) & 15u) << (4 * e)) | ((i4 ? 1u : 0u) << (16 + e));
    }
    nib[p] = n;
    zm[p] = z;
    orl[p] = o;
    const uint32_t row0 = (uint32_t)((int64_t)p * T + t0);
    pb[p] = any_int4 ? row0 * (uint32_t)pitch + base : kOOB;
    // register m, lane l holds run element m*64 + l (out of range past the run)
#pragma unroll
    for (int m = 0; m < RO; ++m) {
      const int i = kWave * m + lane;
      olx[p][m] = i < nrun ? (row0 * (uint32_t)k + (uint32_t)(ilo + i)) * 2u : kOOB;
    }
  }

  // Runs longer than 64 are staged per row in this wave's LDS slice
  // ([shard][256] bf16) and read back by position.
  __shared__ uint16_t run_lds[RO > 1 ? 4 : 1][RO > 1 ? NP * 256 : 1];
  uint16_t* const run = run_lds[RO > 1 ? wave : 0];

  // Row r's loads: the two code dwords and the run of every shard. Rows up
  // to nrows + 1 are loaded (prefetches past the last row): their offsets
  // stay below 2^31, they read inside the tensors or out of range, and
  // nothing of them is stored.
  auto issue = [&](int r, uint32_t (&a0)[NP], uint32_t (&a1)[NP], uint32_t (&av)[NP][RO]) {
    const uint32_t rpo = (uint32_t)r * (uint32_t)pitch;
    const uint32_t roo = (uint32_t)r * (uint32_t)k * 2u;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      a0[p] = __builtin_amdgcn_raw_buffer_load_b32(rp, pb[p] + rpo, 0, kStream);
      a1[p] = __builtin_amdgcn_raw_buffer_load_b32(rp, pb[p] + 4u + rpo, 0, kStream);
#pragma unroll
      for (int m = 0; m < RO; ++m)
        av[p][m] = __builtin_amdgcn_raw_buffer_load_b16(ro, olx[p][m] + roo, 0, 0);
    }
  };
  // y row r from its loaded codes and runs; stored when r is a real row.
  auto row_sum = [&](int r, const uint32_t (&a0)[NP], const uint32_t (&a1)[NP],
                     const uint32_t (&av)[NP][RO]) {
    if (RO > 1) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int m = 0; m < RO; ++m) run[p * 256 + kWave * m + lane] = (uint16_t)av[p][m];
      wave_lds_sync();
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // Unpacked per row: hoisting the fields out of the row loop would take
      // four times the registers.
      settle(nib[p]);
      settle(zm[p]);
      settle(orl[p]);
      const uint64_t wv = (uint64_t)a0[p] | ((uint64_t)a1[p] << 32);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t q = (uint32_t)(wv >> ((nib[p] >> (8 * e)) & 0xFFu)) & 15u;
        const int zi = (int)((zm[p] >> (4 * e)) & 15u);
        const float dq = __fmul_rn((float)((int)q - zi), sc[p][e]);
        const uint32_t rel = (orl[p] >> (8 * e)) & 0xFFu;
        uint32_t bits;
        if (RO == 1)
          bits = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(rel * 4u), (int)av[p][0]);
        else
          bits = run[p * 256 + rel];
        // bf16_to_f32 shifts the upper half out
        const float term = ((zm[p] >> (16 + e)) & 1u) ? dq : bf16_to_f32(bits);
        acc[e] = __fadd_rn(acc[e], term);
      }
    }
    if (RO > 1) wave_lds_sync();   // reads done before the next row's writes
    if (active && r < nrows)
      *reinterpret_cast<float4*>(y + (t0 + r) * H + h0) = make_float4(acc[0], acc[1], acc[2],
                                                                       acc[3]);
  };
  // Two register sets take turns, so a prefetch never has to land before
  // the other set's arithmetic.
  uint32_t a0[NP], a1[NP], av[NP][RO], b0[NP], b1[NP], bv[NP][RO];
  issue(0, a0, a1, av);
  int r = 0;
  do {
    issue(r + 1, b0, b1, bv);
    issue_fence();
    row_sum(r, a0, a1, av);
    issue(r + 2, a0, a1, av);
    issue_fence();
    row_sum(r + 1, b0, b1, bv);
    r += 2;
  } while (r < nrows);
}

// Any shape and alignment: one thread per output element, shards in order.
__global__ __launch_bounds__(256) void decompress_sets_general_kernel(
    const uint8_t* __restrict__ packed, int64_t pitch, const uint16_t* __restrict__ outl,
    int64_t P, int64_t T, int64_t H, int64_t k, const float* __restrict__ scale,
    const uint8_t* __restrict__ zp, const int32_t* __restrict__ fmap, float* __restrict__ y) {
  const int64_t n = T * H;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t t = i / H, h = i % H;
    float acc = 0.0f;
    for (int64_t p = 0; p < P; ++p) {
      const int32_t f = fmap[p * H + h];
      const int64_t row = p * T + t;
      float term;
      if (f >= 0) {
        const uint32_t byte = packed[row * pitch + (f >> 1)];
        const uint32_t q = (f & 1) ? (byte >> 4) : (byte & 15u);
        term = __fmul_rn((float)((int)q - (int)zp[p * H + h]), scale[p * H + h]);
      } else {
        term = bf16_to_f32(outl[row * k + (-1 - f)]);
      }
      acc = __fadd_rn(acc, term);
    }
    y[i] = acc;
  }
}

// Lane-window kernel (P <= 8, H a multiple of 8). A wave-tile is 512
// consecutive features, 8 per lane; a 256-thread block takes 4 adjacent
// tiles of one block of token rows, and all blocks of a row block run on one
// XCD. Unlike the two kernels above it sums with one fma per int4 term (see
// below), so its output matches the sequential formula within fp32 rounding,
// not bit for bit.
//  0. Setup, once per wave, per shard p, from fmap, scale and zero_point:
//     * the lane's int4 features of shard p take consecutive slots from the
//       first one's slot jf, so their codes are the 32 bits at bit 4*jf of
//       the row: one 8-byte load (moved back one dword where it would pass
//       the row's end) and a 64-bit shift give one nibble per slot;
//     * two byte selectors spread those nibbles over the lane's 8 feature
//       positions (v_perm of the low and high nibbles of every byte: even
//       positions into one register, odd into the other, BF16 positions 0);
//     * the scales (0 at BF16 positions) and the per-feature constant
//       -sum_p z*s that seeds the accumulator.
//     The tile's BF16 values: shard p's BF16 features in the tile are a run
//     [ilo_p, ihi_p) of its outlier block, read off fmap at the tile's ends.
//     The runs of all shards, concatenated, are the tile's entries, entry
//     e = r*64 + lane held in register r. Each entry's position in the tile
//     comes from an LDS table that the lanes owning BF16 positions fill.
//  1. Per token row: one code load per shard and kOR entry loads, a ring of
//     kR rows in flight; per shard a shift, the nibble split and two perms,
//     then 8 byte-to-float conversions and 8 fmas.
//  2. The lane writes its 8 sums to one of two wave-private LDS rows, and the
//     entry lanes add their BF16 values there (ds_add_f32, which costs per
//     instruction and per active lane: registers past the tile's entries
//     are skipped and idle lanes masked off). The previous row
//     is read back from the other LDS row after this row's arithmetic, when
//     its adds are done, and stored with two 16-byte stores per lane, each
//     instruction 1 KB of consecutive features. A tile with more entries than
//     its kOR*64 registers adds the rest after the row loop, rereading its
//     rows of y.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kPsWaves = 4;
constexpr int kPsTile = kWave * 8;   // features per wave-tile
constexpr int kPsRing = 4;           // token rows in flight (2 for short batches)
constexpr int kPsRingSmall = 2;
// LDS y row: feature i of the tile at dword ps_pad(i) (4 dwords of padding
// per 32, so the lanes' 32-byte runs spread over the banks).
__device__ __forceinline__ uint32_t ps_pad(uint32_t i) { return i + ((i >> 5) << 2); }
constexpr int kPsRowDw = kPsTile + kPsTile / 8;   // ps_pad(512)

template <int NP, int kOR, int kR>
__global__ __launch_bounds__(256) void decompress_sets_perm_kernel(
    const uint8_t* __restrict__ packed, int pitch, const uint16_t* __restrict__ outl, int64_t T,
    int H, int k, const float* __restrict__ scale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ fmap, float* __restrict__ y, int ntiles, int rows_per_wave,
    int64_t nrowblk, int tbl_dwords) {
  extern __shared__ __align__(16) char smem[];
  int64_t rb, sub;
  const int ntgrp = (ntiles + kPsWaves - 1) / kPsWaves;
  if (!xcd_unit_block(blockIdx.x, ntgrp, nrowblk, &rb, &sub)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = (int)sub * kPsWaves + wave;
  if (c >= ntiles) return;   // no block barrier below
  const int hs = c * kPsTile;
  const int he = min(hs + kPsTile, H);
  const int h0 = hs + 8 * lane;
  const bool active = h0 < he;   // H % 8 == 0: a lane's window is whole or empty
  const int hh = active ? h0 : hs;
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min(T - t0, (int64_t)rows_per_wave);   // >= 1
  float* const ybuf =
      reinterpret_cast<float*>(smem) + (size_t)wave * (2 * kPsRowDw + tbl_dwords);
  uint16_t* const tbl = reinterpret_cast<uint16_t*>(ybuf + 2 * kPsRowDw);
  const uint32_t ya = ps_pad((uint32_t)(8 * lane));   // the lane's 8 sums, 16-byte aligned

  // One descriptor per tensor (the launcher keeps each below 2^30 bytes).
  const rsrc_t rp = make_rsrc(packed, (uint32_t)(NP * T * (int64_t)pitch));
  const rsrc_t ro = make_rsrc(outl, (uint32_t)(NP * T * (int64_t)k * 2));
  const rsrc_t rf = make_rsrc(fmap, (uint32_t)(NP * (int64_t)H * 4));
  const rsrc_t rs = make_rsrc(scale, (uint32_t)(NP * (int64_t)H * 4));
  const rsrc_t rz = make_rsrc(zp, (uint32_t)(NP * (int64_t)H));

  // (a) setup loads: the window's maps, scales and zero points of every
  // shard, and every shard's map at the tile's end
  v4u fa[NP], fb[NP], sa[NP], sb[NP];
  v2u zz[NP];
  uint32_t fend[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint32_t o = (uint32_t)(p * H + hh);
    fa[p] = __builtin_amdgcn_raw_buffer_load_b128(rf, o * 4u, 0, 0);
    fb[p] = __builtin_amdgcn_raw_buffer_load_b128(rf, o * 4u + 16u, 0, 0);
    sa[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, o * 4u, 0, 0);
    sb[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, o * 4u + 16u, 0, 0);
    zz[p] = __builtin_amdgcn_raw_buffer_load_b64(rz, o, 0, 0);
    fend[p] = __builtin_amdgcn_raw_buffer_load_b32(
        rf, he < H ? (uint32_t)(p * H + he) * 4u : kOOB, 0, 0);
  }

  // (b) per-shard lane constants
  uint32_t cofs[NP], csh[NP], selE[NP], selO[NP];
  float sc[NP][8], bias[8];
  int ilo[NP], E[NP + 1];
#pragma unroll
  for (int e = 0; e < 8; ++e) bias[e] = 0.0f;
  E[0] = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int f[8] = {(int)fa[p][0], (int)fa[p][1], (int)fa[p][2], (int)fa[p][3],
                      (int)fb[p][0], (int)fb[p][1], (int)fb[p][2], (int)fb[p][3]};
    int jf = 0x7FFFFFFF;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (f[e] >= 0) jf = min(jf, f[e]);
    const bool any = active && jf != 0x7FFFFFFF;
    uint32_t b = any ? ((uint32_t)jf >> 3) * 4u : 0u;
    uint32_t sh = any ? 4u * ((uint32_t)jf & 7u) : 0u;
    if (b + 8u > (uint32_t)pitch) {   // keep the 8 bytes inside the row (pitch >= 8)
      b -= 4u;
      sh += 32u;
    }
    cofs[p] = any ? b : kOOB;
    csh[p] = sh;
    uint32_t se = 0u, so = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // nibble n of the shifted code word: byte n/2 of the low nibbles
      // (selector n/2) or of the high nibbles (selector 4 + n/2); 12 selects
      // a zero byte
      const int n = f[e] - jf;
      const uint32_t sel = (any && f[e] >= 0) ? ((n & 1) ? 4u + (uint32_t)(n >> 1)
                                                         : (uint32_t)(n >> 1))
                                              : 12u;
      if (e & 1)
        so |= sel << (8 * (e >> 1));
      else
        se |= sel << (8 * (e >> 1));
    }
    selE[p] = se;
    selO[p] = so;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = __uint_as_float(e < 4 ? sa[p][e] : sb[p][e - 4]);
      sc[p][e] = (active && f[e] >= 0) ? s : 0.0f;
      const float z = (float)((zz[p][e >> 2] >> (8 * (e & 3))) & 0xFFu);
      bias[e] = fmaf(-z, sc[p][e], bias[e]);
    }
    // shard p's BF16 features below h: h - fmap[h] where h is int4, -1 - fmap[h]
    // where it is BF16, k at h = H. Lane 0 holds h = hs.
    const int f0 = __builtin_amdgcn_readfirstlane(f[0]);
    const int fe = __builtin_amdgcn_readfirstlane((int)fend[p]);
    ilo[p] = f0 >= 0 ? hs - f0 : -1 - f0;
    const int ihi = he < H ? (fe >= 0 ? he - fe : -1 - fe) : k;
    E[p + 1] = E[p] + (ihi - ilo[p]);
    // entry of each BF16 position of the window: its tile position goes into
    // the table
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (active && f[e] < 0) tbl[E[p] + (-1 - f[e]) - ilo[p]] = (uint16_t)ps_pad(8 * lane + e);
  }
  const int nE = E[NP];
  wave_lds_sync();
  // the entries in registers: outlier-block offset and LDS position (idle
  // lanes load out of range and add nothing)
  uint32_t eoff[kOR], epos[kOR];
#pragma unroll
  for (int r = 0; r < kOR; ++r) {
    const int e = r * kWave + lane;
    int p = 0;
#pragma unroll
    for (int q = 1; q < NP; ++q)
      if (E[q] <= e) p = q;
    const bool ok = e < nE;
    eoff[r] = ok ? (uint32_t)(((int64_t)p * T * k + ilo[p] + (e - E[p])) * 2) : kOOB;
    const uint32_t t = tbl[ok ? e : 0];
    epos[r] = ok ? t : 0u;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) settle(cofs[p]);

  // (c) the ring
  v2u cw[kR][NP];
  uint32_t ev[kR][kOR];
  auto load = [&](int q, int row) {
    const bool ok = row < nrows;   // uniform
    const int64_t rowg = t0 + min(row, nrows - 1);
#pragma unroll
    for (int p = 0; p < NP; ++p)
      cw[q][p] = __builtin_amdgcn_raw_buffer_load_b64(
          rp, ok ? cofs[p] : kOOB, (uint32_t)(((int64_t)p * T + rowg) * pitch), kStream);
#pragma unroll
    for (int r = 0; r < kOR; ++r)
      ev[q][r] = __builtin_amdgcn_raw_buffer_load_b16(ro, ok ? eoff[r] : kOOB,
                                                      (uint32_t)(rowg * k * 2), 0);
  };
  issue_fence();
#pragma unroll
  for (int q = 0; q < kR; ++q) {
    load(q, q);
    issue_fence();
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    settle(csh[p]);
    settle(selE[p]);
    settle(selO[p]);
#pragma unroll
    for (int e = 0; e < 8; ++e) settle(sc[p][e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) settle(bias[e]);

  // y stores: 16 bytes through a per-row descriptor with an immediate-zero
  // scalar offset (the compiler then keeps the data registers of the wide
  // store from being overwritten on the next instruction)
  float* const yrows = y + t0 * H;
  // y is read back from the LDS row in 16-byte chunks: lane l stores chunk l
  // of each half of the tile, so each store instruction writes 1 KB of
  // whole cache lines
  const int hA = hs + 4 * lane, hB = hs + kPsTile / 2 + 4 * lane;
  const uint32_t yoA = hA < he ? (uint32_t)hA * 4u : kOOB;
  const uint32_t yoB = hB < he ? (uint32_t)hB * 4u : kOOB;
  const uint32_t yaA = ps_pad((uint32_t)(4 * lane));
  const uint32_t yaB = ps_pad((uint32_t)(kPsTile / 2 + 4 * lane));
  // (a row outside the wave's stores out of range, so the stores are not
  // under a branch)
  auto store_row = [&](int row, const v4f& lo, const v4f& hi) {
    const bool ok = row >= 0 && row < nrows;   // uniform
    const rsrc_t rr =
        make_rsrc(yrows + (int64_t)min(max(row, 0), nrows - 1) * H, (uint32_t)H * 4u);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, lo), rr, ok ? yoA : kOOB, 0,
                                           kStream);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, hi), rr, ok ? yoB : kOOB, 0,
                                           kStream);
  };

  // Rows alternate between two LDS rows. A row's sums and BF16 adds are
  // issued to one; the previous row is read back from the other only after
  // this row's arithmetic, by when its adds are done, and stored.
  int base = 0;
  do {
#pragma unroll
    for (int q = 0; q < kR; ++q) {
      const int row = base + q;   // base is a multiple of kR, so row & 1 == q & 1
      float* const bcur = ybuf + (q & 1) * kPsRowDw;
      const float* const bprev = ybuf + ((q + 1) & 1) * kPsRowDw;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint64_t w = (uint64_t)cw[q][p][0] | ((uint64_t)cw[q][p][1] << 32);
        const uint32_t code = (uint32_t)(w >> csh[p]);
        const uint32_t lo = code & 0x0F0F0F0Fu;
        const uint32_t hi = (code >> 4) & 0x0F0F0F0Fu;
        uint32_t pe = __builtin_amdgcn_perm(hi, lo, selE[p]);
        uint32_t po = __builtin_amdgcn_perm(hi, lo, selO[p]);
        opaque(pe);
        opaque(po);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          acc[2 * bb] = fmaf((float)((pe >> (8 * bb)) & 0xFFu), sc[p][2 * bb], acc[2 * bb]);
          acc[2 * bb + 1] =
              fmaf((float)((po >> (8 * bb)) & 0xFFu), sc[p][2 * bb + 1], acc[2 * bb + 1]);
        }
      }
      wave_lds_sync();
      const v4f plo = *reinterpret_cast<const v4f*>(bprev + yaA);
      const v4f phi = *reinterpret_cast<const v4f*>(bprev + yaB);
      *reinterpret_cast<v4f*>(bcur + ya) = v4f{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<v4f*>(bcur + ya + 4) = v4f{acc[4], acc[5], acc[6], acc[7]};
      // other lanes add to these sums: the writes go first (LDS executes a
      // wave's operations in order; the fence keeps the compiler's order)
      wave_lds_sync();
      // LDS float adds are costly per instruction and per lane: registers
      // past the tile's entries are skipped, idle lanes masked off
#pragma unroll
      for (int rr = 0; rr < kOR; ++rr)
        if (rr * kWave < nE && rr * kWave + lane < nE)
          __hip_atomic_fetch_add(bcur + epos[rr], bf16_to_f32(ev[q][rr]), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WAVEFRONT);
      // refill the consumed slot (codes and BF16 values) with the row kR ahead
      load(q, row + kR);
      store_row(row - 1, plo, phi);   // row -1 stores out of range
    }
    base += kR;
  } while (base < nrows);
  {   // the loop's last row (base - 1; out of range if past nrows - 1)
    wave_lds_sync();
    const float* const bl = ybuf + ((kR - 1) & 1) * kPsRowDw;
    const v4f llo = *reinterpret_cast<const v4f*>(bl + yaA);
    const v4f lhi = *reinterpret_cast<const v4f*>(bl + yaB);
    store_row(base - 1, llo, lhi);
  }

  if (nE > kOR * kWave) {   // uniform
    // Entries past the registers: wait for the row loop's stores, then add
    // them row by row to y through the LDS row.
    __builtin_amdgcn_s_waitcnt(0);
    for (int row = 0; row < nrows; ++row) {
      const rsrc_t rr = make_rsrc(yrows + (int64_t)row * H, (uint32_t)H * 4u);
      const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(rr, yoA, 0, 0);
      const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(rr, yoB, 0, 0);
      *reinterpret_cast<v4u*>(ybuf + yaA) = lo;
      *reinterpret_cast<v4u*>(ybuf + yaB) = hi;
      wave_lds_sync();
      for (int e0 = kOR * kWave; e0 < nE; e0 += kWave) {
        const int e = e0 + lane;
        int p = 0;
#pragma unroll
        for (int q = 1; q < NP; ++q)
          if (E[q] <= e) p = q;
        const bool ok = e < nE;
        const uint32_t off =
            ok ? (uint32_t)((((int64_t)p * T + t0 + row) * k + ilo[p] + (e - E[p])) * 2) : kOOB;
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(ro, off, 0, 0);
        const uint32_t t = tbl[ok ? e : 0];
        if (ok)
          __hip_atomic_fetch_add(ybuf + t, bf16_to_f32(v), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WAVEFRONT);
      }
      wave_lds_sync();
      const v4f vl = *reinterpret_cast<const v4f*>(ybuf + yaA);
      const v4f vh = *reinterpret_cast<const v4f*>(ybuf + yaB);
      store_row(row, vl, vh);
      wave_lds_sync();
    }
  }
}

template <int NP, int kOR, int kR>
static void launch_sets_perm(const uint8_t* packed, int64_t pitch, const uint16_t* outl,
                             int64_t T, int64_t H, int64_t k, const float* scale,
                             const uint8_t* zp, const int32_t* fmap, float* y, int64_t ntiles,
                             int64_t rpw, int64_t nrowblk, int64_t tbl_dwords, hipStream_t s) {
  const int64_t ntgrp = (ntiles + kPsWaves - 1) / kPsWaves;
  const size_t lds = (size_t)kPsWaves * (2 * kPsRowDw + tbl_dwords) * 4;
  decompress_sets_perm_kernel<NP, kOR, kR>
      <<<(unsigned)xcd_grid(ntgrp, nrowblk), 256, lds, s>>>(
          packed, (int)pitch, outl, T, (int)H, (int)k, scale, zp, fmap, y, (int)ntiles, (int)rpw,
          nrowblk, (int)tbl_dwords);
}

template <int NP>
static void dispatch_sets_perm(bool wide, bool small, const uint8_t* packed, int64_t pitch,
                               const uint16_t* outl, int64_t T, int64_t H, int64_t k,
                               const float* scale, const uint8_t* zp, const int32_t* fmap,
                               float* y, int64_t ntiles, int64_t rpw, int64_t nrowblk,
                               int64_t tbl_dwords, hipStream_t s) {
#define BTQ_PS_ARGS \
  packed, pitch, outl, T, H, k, scale, zp, fmap, y, ntiles, rpw, nrowblk, tbl_dwords, s
  if (wide && small)
    launch_sets_perm<NP, 4, kPsRingSmall>(BTQ_PS_ARGS);
  else if (wide)
    launch_sets_perm<NP, 4, kPsRing>(BTQ_PS_ARGS);
  else if (small)
    launch_sets_perm<NP, 2, kPsRingSmall>(BTQ_PS_ARGS);
  else
    launch_sets_perm<NP, 2, kPsRing>(BTQ_PS_ARGS);
#undef BTQ_PS_ARGS
}

hipError_t launch_decompress_sets(const uint8_t* packed, int64_t pitch, const uint16_t* outl,
                                  int64_t P, int64_t T, int64_t H, int64_t k, const float* scale,
                                  const uint8_t* zp, const int32_t* fmap, float* y,
                                  hipStream_t s) {
  // Lane-window kernel: P <= 8, whole 8-feature windows, more than 2 token
  // rows (for 1 or 2 rows its two dependent setup round trips make it slower
  // than the register kernel: decode at T=1 10.8 against 7.4 us). Every descriptor
  // (message, outlier blocks, maps, scales) spans fewer than 2^30 bytes, and
  // pitch and k below 2^25 keep kOOB plus a row offset from wrapping past
  // 2^32. LDS: the y rows and a table of up to P*min(k, 512) 2-byte entry
  // positions per wave.
  {
    const int64_t ntiles = (H + kPsTile - 1) / kPsTile;
    const int64_t tbl_entries = P * (k < kPsTile ? k : kPsTile);
    const int64_t tbl_dwords = ((tbl_entries + 1) / 2 + 3) / 4 * 4;
    const int64_t lds_max = int64_t(kPsWaves) * (2 * kPsRowDw + tbl_dwords) * 4;
    int64_t rpw = (ntiles * T + 1023) / 1024;
    const bool small = rpw < kPsRing;
    const int64_t ring = small ? kPsRingSmall : kPsRing;
    rpw = (rpw + ring - 1) / ring * ring;
    if (rpw < ring) rpw = ring;
    if (rpw > 64) rpw = 64;
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    const int64_t ntgrp = (ntiles + kPsWaves - 1) / kPsWaves;
    const int64_t lim = int64_t(1) << 30;
    const bool perm = T > 2 && P >= 1 && P <= 8 && H % 8 == 0 && pitch % 4 == 0 && pitch >= 8 &&
                      pitch < (int64_t(1) << 25) && k < (int64_t(1) << 25) &&
                      P * T * (pitch + 8) < lim && P * T * k * 2 < lim && P * H * 4 < lim &&
                      lds_max <= 65536 && (uintptr_t)packed % 4 == 0 &&
                      (uintptr_t)fmap % 16 == 0 && (uintptr_t)scale % 16 == 0 &&
                      (uintptr_t)zp % 8 == 0 && (uintptr_t)y % 16 == 0 &&
                      xcd_grid(ntgrp, nrowblk) < (int64_t(1) << 31);
    if (perm) {
      // entry registers: 2 (128 entries per tile) while the tiles hold at
      // most 64 on average, else 4
      const bool wide = P * k > int64_t(kWave) * ntiles;
#define BTQ_PS_CASE(n)                                                                          \
  case n:                                                                                       \
    dispatch_sets_perm<n>(wide, small, packed, pitch, outl, T, H, k, scale, zp, fmap, y,        \
                          ntiles, rpw, nrowblk, tbl_dwords, s);                                 \
    break;
      switch (P) {
        BTQ_PS_CASE(1)
        BTQ_PS_CASE(2)
        BTQ_PS_CASE(3)
        BTQ_PS_CASE(4)
        BTQ_PS_CASE(5)
        BTQ_PS_CASE(6)
        BTQ_PS_CASE(7)
        BTQ_PS_CASE(8)
      }
#undef BTQ_PS_CASE
      return hipGetLastError();
    }
  }
  // Register kernel: P <= 8, 4-feature lanes. Rows per wave: about 4096
  // waves, 4..32 rows. Every buffer offset (rows * pitch, rows * k * 2)
  // stays below 2^30.
  const int64_t nwin = (H + 255) / 256;
  int64_t rpw = (nwin * T + 4095) / 4096;
  rpw = rpw < 4 ? 4 : rpw > 32 ? 32 : rpw;
  const int64_t nwg = (nwin + 3) / 4;
  const int64_t nrb = (T + rpw - 1) / rpw;
  // One descriptor spans a whole tensor: P*T rows of pitch bytes (and of k
  // BF16 values) below 2^30 bytes, so an offset plus a row stays below 2^31.
  // pitch and k below 2^25 keep kOOB plus (rows per wave + 2) rows from
  // wrapping past 2^32.
  const bool reg = P <= 8 && H % 4 == 0 && H < (int64_t(1) << 30) && pitch % 4 == 0 &&
                   pitch >= 8 && pitch < (int64_t(1) << 25) && k < (int64_t(1) << 25) &&
                   P * T * (pitch + 8) < (int64_t(1) << 30) &&
                   P * T * k * 2 < (int64_t(1) << 30) &&
                   (uintptr_t)packed % 4 == 0 && (uintptr_t)fmap % 16 == 0 &&
                   (uintptr_t)scale % 16 == 0 && (uintptr_t)zp % 4 == 0 &&
                   (uintptr_t)y % 16 == 0 && xcd_grid(nwg, nrb) < (int64_t(1) << 31);
  if (reg) {
    const unsigned blocks = (unsigned)xcd_grid(nwg, nrb);
#define BTQ_SETS(np, ro)                                                                        \
  decompress_sets_reg_kernel<np, ro><<<blocks, 256, 0, s>>>(packed, (int)pitch, outl, T, (int)H, \
                                                            (int)k, scale, zp, fmap, y,          \
                                                            (int)nwin, (int)nwg, (int)rpw, nrb)
#define BTQ_SETS_P(ro)             \
  switch (P) {                     \
    case 1: BTQ_SETS(1, ro); break; \
    case 2: BTQ_SETS(2, ro); break; \
    case 3: BTQ_SETS(3, ro); break; \
    case 4: BTQ_SETS(4, ro); break; \
    case 5: BTQ_SETS(5, ro); break; \
    case 6: BTQ_SETS(6, ro); break; \
    case 7: BTQ_SETS(7, ro); break; \
    default: BTQ_SETS(8, ro); break; \
  }
    // a window's run of one shard's BF16 features is at most min(k, 256) long
    if (k <= kWave) {
      BTQ_SETS_P(1);
    } else if (k <= 2 * kWave) {
      BTQ_SETS_P(2);
    } else {
      BTQ_SETS_P(4);
    }
#undef BTQ_SETS_P
#undef BTQ_SETS
    return hipGetLastError();
  }
  const int64_t nfblk = (H + kSetBlockFeat - 1) / kSetBlockFeat;
  const int64_t nrowblk = (T + kSetRows - 1) / kSetRows;
  const bool fast = H % kSetFeat == 0 && H < (int64_t(1) << 30) && pitch % 4 == 0 &&
                    pitch >= 8 && pitch < (int64_t(1) << 28) && (uintptr_t)packed % 4 == 0 &&
                    (uintptr_t)fmap % 16 == 0 && (uintptr_t)scale % 16 == 0 &&
                    (uintptr_t)zp % 8 == 0 && (uintptr_t)y % 16 == 0 &&
                    nfblk * nrowblk < (int64_t(1) << 31);
  if (fast) {
    decompress_sets_kernel<<<(unsigned)(nfblk * nrowblk), 256, 0, s>>>(
        packed, (int)pitch, outl, P, T, (int)H, (int)k, scale, zp, fmap, y, (int)nfblk);
    return hipGetLastError();
  }
  int64_t blocks = (T * H + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  decompress_sets_general_kernel<<<(unsigned)blocks, 256, 0, s>>>(packed, pitch, outl, P, T, H,
                                                                   k, scale, zp, fmap, y);
  return hipGetLastError();
}

}  // namespace btq
