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

hipError_t launch_decompress_sets(const uint8_t* packed, int64_t pitch, const uint16_t* outl,
                                  int64_t P, int64_t T, int64_t H, int64_t k, const float* scale,
                                  const uint8_t* zp, const int32_t* fmap, float* y,
                                  hipStream_t s) {
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
