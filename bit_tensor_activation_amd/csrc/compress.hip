// Sender side: asymmetric 4-bit quantization of the int4 features, nibble
// packing, and the bit copy of the BF16 features.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Inference
// bullet (selected features keep BF16, the rest go to 4 bits), and section
// "Combating Quantization Errors with Tensor Parallelism" (each device
// quantizes its partial sum before the sum).
//
// Tiles. A wave-tile is 512 int4 slots, 8 per lane, so each lane writes
// exactly one packed dword per token row. The tile also owns the BF16
// features that fall between its slots (TileGeom). Packed rows sit `pitch`
// bytes apart; with a pitch that is a multiple of 128 every tile's 256-byte
// row piece covers whole cache lines, and the lanes past the last slot write
// the row's zero padding.
//
// Ring kernel (the fast path). A 256-thread block takes 4 adjacent tiles of
// one shard's block of token rows, one wave per tile, so the block reads
// about 4 KB of each row in one go. All blocks of a row block run on one XCD
// (xcd_unit_block).
//  0. Setup, once per wave: the lane's 8 feature indices, its BF16 feature
//     index, and the shard's rscale and zero points over the tile's feature
//     span (contiguous 16- and 8-byte loads). Then the first kRing token rows
//     are issued, and only then does the wave wait for the setup values: the
//     span's parameters go through the wave's LDS buffer, where each lane
//     picks its 8 features' (rscale, zero point), before the buffer serves
//     the rows. No block barrier.
//  1. Each ring row arrives as one 16-byte load per lane (the span's first
//     64 chunks); the chunks past 64 (BF16 features and alignment slack)
//     come with one tail load per pair of rows, lanes 0-31 for the first row
//     and 32-63 for the second. kSub = 2 rows at a time are staged in a
//     wave-private LDS buffer and their slots refilled kRing rows ahead.
//  2. Each lane gathers its 8 features from LDS at fixed offsets, quantizes
//     them in the float domain (Quant8), packs 8 nibbles into one dword and
//     stores it: one coalesced 256-byte store per wave and row.
//  3. The tile's BF16 features are copied out of the same LDS buffer, one
//     store per pair of rows (lanes 0-31 the first row's first 32 features,
//     32-63 the second's); features past the 32nd, rare, row by row.
//     (Batching the tail loads and BF16 stores by pairs took the stress shape
//     at k=32 from 481 to 475 us and large prefill from 121.6 to 118.2 us:
//     each is a full wave instruction even when only a few lanes carry data.)
// The staging layout pads 4 bytes after every 16-byte chunk, so lane l's
// features start at dword 5*l and one gather spreads over all banks. All
// global accesses go through per-wave buffer resources: ragged rows, idle
// lanes and surplus chunks become clamped or out-of-range offsets, not
// branches.
//
// Staged kernel: the same tiles for spans too wide for the ring's tail load
// (many BF16 features per tile). A block takes one tile and 4 row blocks.
//
// General kernel. One thread per packed byte and per BF16 value. It serves
// any H, k, pitch, alignment and LDS size.
//
// Per-shard BF16 sets (template flag kPs): cmap [P,H-k] and idx [P,k] hold
// one set per shard, and each (shard, row block) unit offsets them by its
// shard before it derives its tile geometry; nothing else changes.
#include "common.hpp"

namespace btq {

constexpr int kCpWaves = 4;   // waves per 256-thread block, each on its own rows
constexpr int kCpRows = 4;    // token rows staged per step

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pad_byte_off(uint32_t e) {   // element offset -> LDS byte
  return (e >> 3) * 20u + (e & 7u) * 2u;
}

__device__ __forceinline__ uint32_t quant4(uint32_t bits16, float r, float z) {
  const float v = __fmul_rn(bf16_to_f32(bits16), r);
  const float q = __builtin_amdgcn_fmed3f(rintf(v) + z, 0.0f, 15.0f);
  return (uint32_t)q;
}

// A lane's 8 codes, quant4 of each feature, packed into one dword with
// fewer instructions: the rounding, the zero point and the conversion to an
// integer all stay in the float domain. With M = 1.5 * 2^23, fl(v + M) is
// M + rint(v), rounded half to even, whenever |v| < 2^22; every other v
// lands outside [M - z, M + 15 - z], on the side its sign gives. Clamping
// fl(v + M) to those bounds therefore equals M - z + clamp(rint(v) + z, 0,
// 15), and its bit pattern is 0x4B400000 + (q - z), an integer. Adding each
// feature's pattern, shifted to its nibble, to the constant
// -sum_e (0x4B400000 - z_e) << 4e leaves exactly the packed codes (mod
// 2^32, with no carries between nibbles in the result).
constexpr float kQMagic = 12582912.0f;   // 1.5 * 2^23, bits 0x4B400000
// kLean: the zero point is added by a second float add, fl(fl(v + M) + z),
// and the sum clamped to the constant bounds [M, M + 15]. For |v| < 2^22 the
// add is exact (the sum stays below 2^24); a larger v stays past its bound
// (v >= 2^22 gives at least M + 2^22, v <= -2^22 at most 2^23 + 15 < M). The
// pattern is then 0x4B400000 + q and the constant -sum_e 0x4B400000 << 4e.
// One more instruction per feature and 9 fewer registers: the widest-span
// ring kernel keeps 4 waves per SIMD with it.
template <bool kLean>
struct Quant8 {
  float lo[kLean ? 1 : 8], hi[kLean ? 1 : 8];   // M - z, M + 15 - z
  float zf[kLean ? 8 : 1];                      // z
  uint32_t k;   // -sum_e (0x4B400000 - z_e) << 4e  (kLean: -sum_e 0x4B400000 << 4e)

  __device__ __forceinline__ void init(const float (&z)[8]) {
    k = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (kLean) {
        zf[e] = z[e];
        k -= 0x4B400000u << (4 * e);
      } else {
        lo[e] = kQMagic - z[e];
        hi[e] = kQMagic + (15.0f - z[e]);
        k -= (0x4B400000u - (uint32_t)z[e]) << (4 * e);
      }
    }
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (kLean) {
        settle(zf[e]);
      } else {
        settle(lo[e]);
        settle(hi[e]);
      }
    }
    settle(k);
  }
  // u: the 8 features' bf16 bits
  __device__ __forceinline__ uint32_t pack(const uint32_t (&u)[8], const float (&rs)[8]) const {
    uint32_t w = k;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = __fmul_rn(bf16_to_f32(u[e]), rs[e]);
      float c;
      if constexpr (kLean)
        c = __builtin_amdgcn_fmed3f(__fadd_rn(__fadd_rn(v, kQMagic), zf[e]), kQMagic,
                                    kQMagic + 15.0f);
      else
        c = __builtin_amdgcn_fmed3f(__fadd_rn(v, kQMagic), lo[e], hi[e]);
      const uint32_t b = __float_as_uint(c);
      // one shift-and-add per feature (left to itself the compiler spends
      // three instructions on every two)
      if (e == 0)
        w += b;
      else
        asm("v_lshl_add_u32 %0, %1, %2, %0" : "+v"(w) : "v"(b), "n"(4 * e));
    }
    return w;
  }
};

// Per-feature parameters of one shard over a tile's feature span
// [a0, a0 + 8*nch): rscale as 16-byte chunks of 4 floats, zero points as
// 8-byte chunks of 8 bytes. kR, kZ: chunks per lane that cover the widest
// span the kernel takes. A chunk past the span loads out of range (zeros).
template <int kR, int kZ>
struct SpanParams {
  v4u r[kR];
  uint64_t z[kZ];

  __device__ __forceinline__ void load(const float* rscale, const uint8_t* zp, int nch,
                                       int lane) {
    const rsrc_t rr = make_rsrc(rscale, (uint32_t)nch * 32u);
    const rsrc_t rz = make_rsrc(zp, (uint32_t)nch * 8u);
#pragma unroll
    for (int m = 0; m < kR; ++m)
      r[m] = __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)(lane + kWave * m) * 16u, 0, 0);
#pragma unroll
    for (int m = 0; m < kZ; ++m) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(rz, (uint32_t)(lane + kWave * m) * 8u,
                                                          0, 0);
      z[m] = (uint64_t)t[0] | ((uint64_t)t[1] << 32);
    }
  }

  // Writes the span to LDS (rscale floats at byte 0, zero-point bytes at
  // byte 32*nch; 40*nch bytes in all), then reads the lane's 8 features
  // hh[e] (each in the span) back as (rscale, zero point as a float).
  __device__ __forceinline__ void pick(char* buf, int nch, int lane, int a0, const int hh[8],
                                       float rs[8], float zf[8]) const {
#pragma unroll
    for (int m = 0; m < kR; ++m) {
      const int c = lane + kWave * m;
      if (c < 2 * nch) *reinterpret_cast<v4u*>(buf + 16 * c) = r[m];
    }
#pragma unroll
    for (int m = 0; m < kZ; ++m) {
      const int c = lane + kWave * m;
      if (c < nch) *reinterpret_cast<uint64_t*>(buf + 32 * nch + 8 * c) = z[m];
    }
    wave_lds_sync();
    const float* pf = reinterpret_cast<const float*>(buf);
    const uint8_t* pb = reinterpret_cast<const uint8_t*>(buf + 32 * nch);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      rs[e] = pf[hh[e] - a0];
      zf[e] = (float)pb[hh[e] - a0];
    }
    wave_lds_sync();   // the buffer serves the token rows next
  }
};

// Staged kernel. LDS: 4 waves x kCpRows staging buffers of buf_bytes.
// kPs: idx [P,k] and cmap [P,Hq] hold one BF16 set per shard.
template <int kMaxChunks, bool kPs>
__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ x, int64_t T, int H, int Hq, int k, int ntiles,
    int rows_per_wave, int64_t nrowblk, int64_t ngroups, int buf_bytes,
    int64_t P, const float* __restrict__ rscale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap,
    uint8_t* __restrict__ packed, int pitch, uint16_t* __restrict__ outl) {
  extern __shared__ __align__(16) char smem[];
  // unit = (shard, row group); its ntiles blocks run on one XCD
  int64_t unit, sub;
  if (!xcd_unit_block(blockIdx.x, ntiles, P * ngroups, &unit, &sub)) return;
  const int c = (int)sub;
  const int64_t rg = unit % ngroups;
  const int64_t p = unit / ngroups;
  if (kPs) {   // this shard's own set
    cmap += p * Hq;
    idx += p * k;
  }
  const TileGeom g = tile_geom(cmap, c, ntiles, Hq, H);
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep
  // everything derived from it (rows, descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rb = rg * kCpWaves + wave;
  if (rb >= nrowblk) return;   // no rows for this wave (no block barrier below)
  const int a0 = g.hs & ~7;
  const int nch = (((g.he + 7) & ~7) - a0) >> 3;   // 16-byte chunks in the span
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min(T - t0, (int64_t)rows_per_wave);
  const int64_t row0 = p * T + t0;
  char* const buf = smem + (size_t)wave * kCpRows * buf_bytes;

  // This wave's rows of x, packed and outliers, as buffer resources.
  const rsrc_t rx = make_rsrc(x + row0 * H, (uint32_t)nrows * (uint32_t)H * 2u);
  const rsrc_t rp = make_rsrc(packed + row0 * pitch, (uint32_t)nrows * (uint32_t)pitch);
  const rsrc_t ro = make_rsrc(outl + row0 * k, (uint32_t)nrows * (uint32_t)k * 2u);
  const rsrc_t rc = make_rsrc(cmap, (uint32_t)Hq * 4u);

  // Chunk m of lane l is span chunk l + 64m. Surplus lanes load out of range
  // (no memory traffic) and write nothing.
  uint32_t gx[kMaxChunks], lx[kMaxChunks];
#pragma unroll
  for (int m = 0; m < kMaxChunks; ++m) {
    const int ci = lane + kWave * m;
    gx[m] = (ci < nch) ? (uint32_t)(a0 + 8 * ci) * 2u : kOOB;
    lx[m] = (uint32_t)ci * 20u;
  }
  const uint32_t rowb = (uint32_t)H * 2u;

  v4u v[kCpRows][kMaxChunks];
  // The lane's offset stays in one VGPR per chunk; the row offset is uniform
  // and rides in the instruction's SGPR offset. No per-row address math, and
  // no register that a load in flight still owns is rewritten.
  auto load_rows = [&](int s) {
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
      const uint32_t ro_ = (uint32_t)min(s + r, nrows - 1) * rowb;
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m)
        v[r][m] = __builtin_amdgcn_raw_buffer_load_b128(rx, gx[m], ro_, kStream);
    }
  };
  // Per-lane constants for the whole tile, loaded before the first rows
  // (the vector-memory counter retires in order). Idle lanes (past the end
  // of a partial last tile) read valid indices and store out of range.
  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  const int jj = active ? j0 : g.jstart;
  const v4u hA = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u, 0, 0);
  const v4u hB = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u + 16u, 0, 0);
  // the shard's parameters over the span (at most 4*kWave chunks of 8 features)
  SpanParams<8, 4> sp;
  sp.load(rscale + p * H + a0, zp + p * H + a0, nch, lane);
  load_rows(0);
  const int hh[8] = {(int)hA[0], (int)hA[1], (int)hA[2], (int)hA[3],
                     (int)hB[0], (int)hB[1], (int)hB[2], (int)hB[3]};
  float rs[8], zf[8];
  sp.pick(buf, nch, lane, a0, hh, rs, zf);   // (kCpRows*buf_bytes >= 40*nch)
  Quant8<false> qz;
  qz.init(zf);
  uint32_t ad[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ad[e] = pad_byte_off((uint32_t)(hh[e] - a0));
  // (lanes past the last slot write the row's zero padding, up to the pitch)
  const uint32_t st_off = ((j0 >> 1) + 4 <= pitch) ? (uint32_t)(j0 >> 1) : kOOB;
  const int nout_it = (g.nout + kWave - 1) / kWave;   // uniform
  uint32_t oad = 0;
  if (g.nout > 0) oad = pad_byte_off((uint32_t)(idx[g.ilo + min(lane, g.nout - 1)] - a0));
  const uint32_t o_off = (lane < g.nout) ? (uint32_t)(g.ilo + lane) * 2u : kOOB;

  for (int s = 0; s < nrows; s += kCpRows) {
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m) {
        // Surplus lanes skip the write: many lanes storing to one LDS address
        // serialize on its bank.
        if (lane + kWave * m < nch) {
          uint32_t* d = reinterpret_cast<uint32_t*>(buf + r * buf_bytes + lx[m]);
          d[0] = v[r][m][0];
          d[1] = v[r][m][1];
          d[2] = v[r][m][2];
          d[3] = v[r][m][3];
        }
      }
    }
    wave_lds_sync();
    if (s + kCpRows < nrows) load_rows(s + kCpRows);   // in flight during the compute below
    // all gathers of the step first, then the math: one LDS round trip, not 32
    uint32_t u[kCpRows][8];
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        u[r][e] = *reinterpret_cast<const uint16_t*>(buf + r * buf_bytes + ad[e]);
    }
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
      const int row = s + r;
      if (row >= nrows) break;
      uint32_t w = qz.pack(u[r], rs);
      w = active ? w : 0u;   // past the last slot: the row's zero padding
      __builtin_amdgcn_raw_buffer_store_b32(w, rp, st_off, (uint32_t)row * (uint32_t)pitch, kStream);
    }
    for (int it = 0; it < nout_it; ++it) {
      const int i = lane + kWave * it;
      const uint32_t o =
          (it == 0) ? oad : pad_byte_off((uint32_t)(idx[g.ilo + min(i, g.nout - 1)] - a0));
      const uint32_t off =
          (it == 0) ? o_off : ((i < g.nout) ? (uint32_t)(g.ilo + i) * 2u : kOOB);
#pragma unroll
      for (int r = 0; r < kCpRows; ++r) {
        const int row = s + r;
        if (row >= nrows) break;
        const uint16_t b16 = *reinterpret_cast<const uint16_t*>(buf + r * buf_bytes + o);
        __builtin_amdgcn_raw_buffer_store_b16(b16, ro, off, (uint32_t)row * (uint32_t)k * 2u, 0);
      }
    }
    wave_lds_sync();
  }
}

// Ring kernel. Each wave keeps kRing token rows in flight in registers and
// stages kSub of them at a time through a small LDS buffer. Rows past the
// wave's last row load and store out of range, so every trip of the loop
// issues the same memory instructions and the compiler can count exactly
// which loads it must wait for.
constexpr int kRing = 8;        // token rows in flight per wave
constexpr int kRingSmall = 2;   // the same for short batches (decode): more, shorter waves
constexpr int kSub = 2;         // token rows staged in LDS per sub-step

// Staging bytes per row for a tail of kRemDw dwords per lane: 64 + 16*kRemDw
// chunks of 20 bytes. A compile-time stride lets the row offset ride in the
// LDS instruction's immediate field.
template <int kRemDw>
constexpr int ring_row_bytes() { return (kWave + 16 * kRemDw) * 20; }

template <int kRemDw, int kR, bool kPs>
__global__ __launch_bounds__(256) void compress_ring_kernel(
    const uint16_t* __restrict__ x, int64_t T, int H, int Hq, int k, int ntiles,
    int rows_per_wave, int64_t nrowblk, int ntgrp, int64_t P,
    const float* __restrict__ rscale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap,
    uint8_t* __restrict__ packed, int pitch, uint16_t* __restrict__ outl) {
  constexpr int buf_bytes = ring_row_bytes<kRemDw>();
  static_assert(kSub == 2 && kR % 2 == 0, "tails and BF16 copies go by pairs of rows");
  extern __shared__ __align__(16) char smem[];
  // unit = (shard, row block); its ntgrp blocks of 4 adjacent tiles run on
  // one XCD
  int64_t unit, sub;
  if (!xcd_unit_block(blockIdx.x, ntgrp, P * nrowblk, &unit, &sub)) return;
  const int64_t rb = unit % nrowblk;
  const int64_t p = unit / nrowblk;
  if (kPs) {   // this shard's own set
    cmap += p * Hq;
    idx += p * k;
  }
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep
  // everything derived from it (rows, descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = (int)sub * kCpWaves + wave;
  if (c >= ntiles) return;   // past the last tile (no block barrier below)
  const TileGeom g = tile_geom(cmap, c, ntiles, Hq, H);
  const int a0 = g.hs & ~7;
  const int nch = (((g.he + 7) & ~7) - a0) >> 3;   // 16-byte chunks in the span
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min(T - t0, (int64_t)rows_per_wave);
  const int64_t row0 = p * T + t0;
  char* const buf = smem + (size_t)wave * kSub * buf_bytes;

  const rsrc_t rx = make_rsrc(x + row0 * H, (uint32_t)nrows * (uint32_t)H * 2u);
  const rsrc_t rp = make_rsrc(packed + row0 * pitch, (uint32_t)nrows * (uint32_t)pitch);
  const rsrc_t ro = make_rsrc(outl + row0 * k, (uint32_t)nrows * (uint32_t)k * 2u);
  const rsrc_t rc = make_rsrc(cmap, (uint32_t)Hq * 4u);

  // main chunk: lane l loads span chunk l (zeros past the span)
  const uint32_t gmain = (lane < nch) ? (uint32_t)(a0 + 8 * lane) * 2u : kOOB;
  const uint32_t lmain = (uint32_t)lane * 20u;
  // tail: per pair of rows, the span past chunk 64; lanes 0-31 take the
  // pair's first row and 32-63 its second. Each tail load instruction gives
  // a row's 32 lanes kTW contiguous dwords each (instruction i: dwords
  // 32*kTW*i + kTW*(lane & 31) ...). The launcher guarantees the tail fits
  // (nch - 64 <= 16*kRemDw chunks = 32 lanes x kTD dwords).
  constexpr int kTD = 2 * (kRemDw > 0 ? kRemDw : 1);   // tail dwords per lane and pair
  constexpr int kTW = kTD == 2 ? 2 : 4;                // dwords per lane and instruction
  constexpr int kTI = kTD / kTW;                       // tail instructions per pair
  const int half = lane >> 5;
  const int ntail = max(nch - kWave, 0) * 4;
  const uint32_t rowb = (uint32_t)H * 2u;
  auto tail_dw = [&](int i) { return kTW * (lane & 31) + 32 * kTW * i; };
  uint32_t gtail[kTI];
#pragma unroll
  for (int i = 0; i < kTI; ++i)
    gtail[i] = (tail_dw(i) < ntail)
                   ? (uint32_t)(a0 + 8 * kWave + 2 * tail_dw(i)) * 2u + (uint32_t)half * rowb
                   : kOOB;

  v4u vm[kR];
  uint32_t vt[kR / 2][kTD];
  // (The tail loads carry no streaming hint: their lines begin the next
  // tile's span, which another wave reads too; without the hint the L2 keeps
  // them, and stress k=32 took 470 instead of 475 us, 7B 32.8 instead of
  // 33.5 us. The main loads keep it: without it 7B took 35.7 us.)
  auto load = [&](int q, int row) {
    const bool ok = row < nrows;   // uniform
    const uint32_t so = (uint32_t)min(row, nrows - 1) * rowb;
    vm[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? gmain : kOOB, so, kStream);
    if constexpr (kRemDw > 0) {
      if ((q & 1) == 0) {   // the pair (row, row + 1): q is a compile-time slot
        const bool ok2 = row + half < nrows;
#pragma unroll
        for (int i = 0; i < kTI; ++i) {
          const uint32_t o = ok2 ? gtail[i] : kOOB;
          if constexpr (kTW == 2) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(rx, o, so, 0);
            vt[q / 2][0] = t[0];
            vt[q / 2][1] = t[1];
          } else {
            const v4u t = __builtin_amdgcn_raw_buffer_load_b128(rx, o, so, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) vt[q / 2][4 * i + j] = t[j];
          }
        }
      }
    }
  };

  // Setup loads first, ring loads second: the vector-memory counter retires
  // in order, so waiting for a setup load never waits for the ring.
  // (a) the lane's 8 feature indices and its BF16 feature index
  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  const int jj = active ? j0 : g.jstart;
  const v4u hA = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u, 0, 0);
  const v4u hB = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u + 16u, 0, 0);
  const rsrc_t ri_ = make_rsrc(idx, (uint32_t)k * 4u);
  const uint32_t oh = __builtin_amdgcn_raw_buffer_load_b32(
      ri_, (g.nout > 0) ? (uint32_t)(g.ilo + min(lane & 31, g.nout - 1)) * 4u : kOOB, 0, 0);
  // (b) the shard's parameters over the span: its nch <= 64 + 16*kRemDw
  // chunks of 8 features take 2*nch rscale and nch zero-point chunks
  constexpr int kNchMax = kWave + 16 * kRemDw;
  SpanParams<(2 * kNchMax + kWave - 1) / kWave, (kNchMax + kWave - 1) / kWave> sp;
  sp.load(rscale + p * H + a0, zp + p * H + a0, nch, lane);
  // (c) the ring: the first kR rows. Unconditional: a branch around it
  // would make the compiler assume at the join that these loads might not
  // exist, and wait for the ring when it waits for the setup loads.
  // (one fence per row keeps the rows in issue order: the loop consumes
  // them oldest first)
  issue_fence();
#pragma unroll
  for (int q = 0; q < kR; ++q) {
    load(q, q);
    issue_fence();
  }

  const int hh[8] = {(int)hA[0], (int)hA[1], (int)hA[2], (int)hA[3],
                     (int)hB[0], (int)hB[1], (int)hB[2], (int)hB[3]};
  // the lane's 8 (rscale, zero point) pairs, through the staging buffer
  // (kSub*buf_bytes = 40*kNchMax bytes: it holds any span's parameters)
  float rs[8], zf[8];
  sp.pick(buf, nch, lane, a0, hh, rs, zf);
  Quant8<(kRemDw > 2)> qz;
  qz.init(zf);
  uint32_t ad[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ad[e] = pad_byte_off((uint32_t)(hh[e] - a0));
    settle(rs[e]);
  }
  qz.settle_all();
  // (lanes past the last slot write the row's zero padding, up to the pitch)
  const uint32_t st_off = ((j0 >> 1) + 4 <= pitch) ? (uint32_t)(j0 >> 1) : kOOB;
  // BF16 copy, per pair of rows: lane l takes feature (l & 31) of the tile's
  // BF16 features in row `half` of the pair.
  // (used unconditionally: a load whose only use sits under a branch gets
  // sunk below the ring prologue, and its wait would then drain the ring;
  // with no BF16 feature oh reads 0 and the clamp keeps the offset in range)
  const uint32_t oad = pad_byte_off((uint32_t)max((int)oh - a0, 0)) + (uint32_t)(half * buf_bytes);
  const uint32_t o_off = ((lane & 31) < g.nout)
                             ? (uint32_t)(g.ilo + (lane & 31)) * 2u + (uint32_t)(half * k) * 2u
                             : kOOB;

  // nrows >= 1 here. The do-while has no entry guard: a guarded loop lets the
  // compiler sink the prologue loads below the guard, past the point where
  // the setup registers settle.
  int base = 0;
  do {
#pragma unroll
    for (int sb = 0; sb < kR / kSub; ++sb) {
      // stage kSub rows (the main chunk of lanes past the span lands in
      // unused chunk slots of the buffer; tail dwords past the span skip)
#pragma unroll
      for (int r = 0; r < kSub; ++r) {
        const int q = sb * kSub + r;
        uint32_t* dm = reinterpret_cast<uint32_t*>(buf + r * buf_bytes + lmain);
        dm[0] = vm[q][0];
        dm[1] = vm[q][1];
        dm[2] = vm[q][2];
        dm[3] = vm[q][3];
      }
      if constexpr (kRemDw > 0) {   // the pair's tails: each lane into its row's buffer
        char* bt = buf + half * buf_bytes;
#pragma unroll
        for (int i = 0; i < kTI; ++i) {
#pragma unroll
          for (int j = 0; j < kTW; ++j) {
            const int d = tail_dw(i) + j;
            if (d < ntail)
              *reinterpret_cast<uint32_t*>(bt + (kWave + (d >> 2)) * 20 + (d & 3) * 4) =
                  vt[sb][kTW * i + j];
          }
        }
      }
      wave_lds_sync();
      // refill the staged slots with the rows kR ahead
#pragma unroll
      for (int r = 0; r < kSub; ++r) load(sb * kSub + r, base + kR + sb * kSub + r);
      uint32_t u[kSub][8];
#pragma unroll
      for (int r = 0; r < kSub; ++r) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          u[r][e] = *reinterpret_cast<const uint16_t*>(buf + r * buf_bytes + ad[e]);
      }
#pragma unroll
      for (int r = 0; r < kSub; ++r) {
        const int row = base + sb * kSub + r;
        const bool ok = row < nrows;   // uniform
        const uint32_t rr = (uint32_t)min(row, nrows - 1);
        uint32_t w = qz.pack(u[r], rs);
        w = active ? w : 0u;   // past the last slot: the row's zero padding
        __builtin_amdgcn_raw_buffer_store_b32(w, rp, ok ? st_off : kOOB, rr * (uint32_t)pitch,
                                              kStream);
        // a tile's BF16 features past the 32nd (uniform, rare): row by row
        for (int i = lane + 32; i - lane < g.nout; i += kWave) {
          const uint32_t o = pad_byte_off((uint32_t)(idx[g.ilo + min(i, g.nout - 1)] - a0));
          const uint16_t v16 = *reinterpret_cast<const uint16_t*>(buf + r * buf_bytes + o);
          const uint32_t off = (ok && i < g.nout) ? (uint32_t)(g.ilo + i) * 2u : kOOB;
          __builtin_amdgcn_raw_buffer_store_b16(v16, ro, off, rr * (uint32_t)k * 2u, 0);
        }
      }
      {   // the pair's first 32 BF16 features of each row, one store
        const int rowa = base + sb * kSub;
        const uint16_t b16 = *reinterpret_cast<const uint16_t*>(buf + oad);
        __builtin_amdgcn_raw_buffer_store_b16(b16, ro, (rowa + half < nrows) ? o_off : kOOB,
                                              (uint32_t)min(rowa, nrows - 1) * (uint32_t)k * 2u, 0);
      }
      wave_lds_sync();
    }
    base += kR;
  } while (base < nrows);
}

template <bool kPs>
__global__ __launch_bounds__(256) void compress_general_kernel(
    const uint16_t* __restrict__ x, int64_t P, int64_t T, int64_t H, int64_t k, int64_t Hq,
    int64_t Bq, const float* __restrict__ rscale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cmap, uint8_t* __restrict__ packed, int64_t pitch,
    uint16_t* __restrict__ outl) {
  const int64_t n1 = P * T * pitch;
  const int64_t n2 = P * T * k;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1 + n2; i += stride) {
    if (i < n1) {
      const int64_t row = i / pitch, byte = i % pitch;
      const int64_t p = row / T;
      const int64_t j = 2 * byte;
      uint32_t q = 0;   // padding bytes past the codes stay zero
      if (byte < Bq) {
        const int32_t* cm = cmap + (kPs ? p * Hq : 0);
        const int64_t h0 = cm[j];
        q = quant4(x[row * H + h0], rscale[p * H + h0], (float)zp[p * H + h0]);
        if (j + 1 < Hq) {
          const int64_t h1 = cm[j + 1];
          q |= quant4(x[row * H + h1], rscale[p * H + h1], (float)zp[p * H + h1]) << 4;
        }
      }
      packed[i] = (uint8_t)q;
    } else {
      const int64_t ii = i - n1;
      const int64_t row = ii / k, o = ii % k;
      outl[ii] = x[row * H + idx[(kPs ? (row / T) * k : 0) + o]];
    }
  }
}

// Rows per wave: about 8192 waves over the chip (32 per CU), a multiple of
// the staging depth, 4..64 rows.
static int pick_rows_per_wave(int64_t tile_waves, int64_t T) {
  int64_t rpw = (tile_waves * T + 8191) / 8192;
  rpw = (rpw + kCpRows - 1) / kCpRows * kCpRows;
  if (rpw < kCpRows) rpw = kCpRows;
  if (rpw > 64) rpw = 64;
  return (int)rpw;
}

template <bool kPs>
static hipError_t launch_compress_t(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                                    const float* rscale, const uint8_t* zp, const int32_t* idx,
                                    const int32_t* cmap,
                                    uint8_t* packed, int64_t pitch, uint16_t* outl,
                                    hipStream_t s) {
  const int64_t Hq = H - k;
  const int64_t Bq = (Hq + 1) / 2;
  const int64_t ntiles64 = (Hq + kTileSlots - 1) / kTileSlots;
  // A tile's feature span holds its 512 slots plus the BF16 features between
  // them: at most min(H, 512 + k) features. Staging adds 14 of alignment slack.
  const int64_t span = (H < kTileSlots + k ? H : kTileSlots + k);
  const int64_t nch_max = (span + 16 + 7) / 8;
  const int buf_bytes = (int)((nch_max * 20 + 15) / 16 * 16);
  const size_t lds = (size_t)kCpWaves * kCpRows * buf_bytes;
  // The per-wave buffer resources span at most 64 rows of H bf16 values:
  // H < 2^24 keeps them below 2^31 bytes.
  const bool fast = Hq > 0 && H % 8 == 0 && Hq % 8 == 0 && H < (int64_t(1) << 24) &&
                    (uintptr_t)x % 16 == 0 && (uintptr_t)packed % 4 == 0 &&
                    (uintptr_t)rscale % 4 == 0 && (uintptr_t)zp % 4 == 0 &&
                    nch_max <= 4 * kWave && lds <= 65536 &&
                    // the pitch: dword stores, and the lanes of the last
                    // tile reach every padding byte
                    pitch % 4 == 0 && pitch <= ntiles64 * (kTileSlots / 2);
  // Ring kernel: span chunks past 64 must fit the tail load (16 chunks per
  // tail dword per lane).
  const int64_t tail = nch_max > kWave ? nch_max - kWave : 0;
  const int rem_dw = tail == 0 ? 0 : tail <= 16 ? 1 : tail <= 32 ? 2 : tail <= 64 ? 4 : -1;
  const int ring_buf = (kWave + 16 * (rem_dw > 0 ? rem_dw : 0)) * 20;
  const size_t ring_lds = (size_t)kCpWaves * kSub * ring_buf;
  if (fast && rem_dw >= 0 && ring_lds <= 65536) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    // Rows per wave: enough for about 4096 waves (16 per CU, one resident
    // generation) up to 32 rows; larger batches run several generations of
    // 16-row waves, whose short lifetimes keep the end of the launch
    // balanced. A multiple of the ring depth; batches too short to give every
    // wave a full 8-row ring take the 2-row ring.
    int64_t rpw64 = (P * ntiles * T + 4095) / 4096;
    if (rpw64 > 32) rpw64 = 16;
    const int ring = rpw64 < kRing ? kRingSmall : kRing;
    rpw64 = (rpw64 + ring - 1) / ring * ring;
    if (rpw64 < ring) rpw64 = ring;
    const int rpw = (int)rpw64;
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    const int ntgrp = (ntiles + kCpWaves - 1) / kCpWaves;
    const unsigned blocks = (unsigned)xcd_grid(ntgrp, P * nrowblk);
#define BTQ_RING(n, r)                                                                    \
  compress_ring_kernel<n, r, kPs><<<blocks, 256, ring_lds, s>>>(                           \
      x, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, ntgrp, P, rscale, zp, idx, cmap,   \
      packed, (int)pitch, outl)
#define BTQ_RING_R(n) \
  if (ring == kRing) BTQ_RING(n, kRing); else BTQ_RING(n, kRingSmall);
    switch (rem_dw) {
      case 0: BTQ_RING_R(0); break;
      case 1: BTQ_RING_R(1); break;
      case 2: BTQ_RING_R(2); break;
      default: BTQ_RING_R(4); break;
    }
#undef BTQ_RING_R
#undef BTQ_RING
    return hipGetLastError();
  }
  if (fast) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    const int rpw = pick_rows_per_wave(P * ntiles, T);
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    const int64_t ngroups = (nrowblk + kCpWaves - 1) / kCpWaves;
    const int64_t blocks = xcd_grid(ntiles, P * ngroups);
    if (nch_max <= 2 * kWave)
      compress_kernel<2, kPs><<<(unsigned)blocks, 256, lds, s>>>(
          x, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, ngroups, buf_bytes, P, rscale,
          zp, idx, cmap, packed, (int)pitch, outl);
    else
      compress_kernel<4, kPs><<<(unsigned)blocks, 256, lds, s>>>(
          x, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, ngroups, buf_bytes, P, rscale,
          zp, idx, cmap, packed, (int)pitch, outl);
    return hipGetLastError();
  }
  const int64_t n = P * T * (pitch + k);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  compress_general_kernel<kPs><<<(unsigned)blocks, 256, 0, s>>>(x, P, T, H, k, Hq, Bq, rscale, zp,
                                                                idx, cmap, packed, pitch, outl);
  return hipGetLastError();
}

hipError_t launch_compress(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                           const float* rscale, const uint8_t* zp, const int32_t* idx,
                           const int32_t* cmap, uint8_t* packed, int64_t pitch, uint16_t* outl,
                           bool per_shard, hipStream_t s) {
  return per_shard ? launch_compress_t<true>(x, P, T, H, k, rscale, zp, idx, cmap, packed, pitch,
                                             outl, s)
                   : launch_compress_t<false>(x, P, T, H, k, rscale, zp, idx, cmap, packed, pitch,
                                              outl, s);
}

}  // namespace btq
