// Receiver side: fused dequantize of P shards' messages and fp32 sum.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Inference
// bullet (after communication every tensor is converted back and the
// devices' values are summed).
//
// Fast kernel, specialised on the shard count (1..8). A wave-tile is the
// sender's 512 int4 slots, 8 per lane. A 256-thread block takes 4 adjacent
// tiles of one block of token rows, one wave per tile; all blocks of a row
// block run on one XCD, so the partial cache lines of y at tile boundaries
// merge in one L2.
//  0. Setup, once per wave: the lane's 8 slots' scales for every shard and
//     their constant -sum_p z*s (which seeds the accumulator) from the
//     decoder table, in slot order (32 contiguous bytes per table row); the
//     lane's 8 feature indices; its BF16 feature index. Then the first
//     kDqRing rows are issued, and only then does the wave wait for the setup
//     values. No LDS staging of parameters and no block barrier.
//  1. Per token row, each lane holds one packed dword per shard, so each
//     packed byte is read from HBM exactly once, in coalesced 256-byte wave
//     loads. The tile's BF16 values of all shards fill kOR registers across
//     the wave, one lane per (shard, feature). A ring of kDqRing rows stays
//     in flight, and consumed slots reload kDqRing rows ahead.
//  2. A low nibble converts with one byte-to-float instruction. A high nibble
//     is masked in place (16*q) and meets a scale pre-divided by 16, which is
//     exact. Each term is one fma. For a BF16 feature, the lane that owns it
//     fetches its shards' values across lanes (ds_bpermute) and adds them in
//     shard order from 0. A tile with more BF16 values than kOR registers
//     hold sums them after the row loop instead.
//  3. The outputs scatter to their feature positions in a wave-private LDS
//     row. The wave then writes the tile's span of y with 16-byte stores
//     (whole aligned chunks) and one dword store for the at most 6 ragged
//     features at its ends.
//
// General kernel: one thread per (token, slot) and per (token, BF16 feature).
// It evaluates term = fl(q - z) * s and adds the terms in shard order, for
// any P, H, k, pitch and alignment. Both kernels read the decoder table
// [2P+1, Hq]: rows 0..P-1 scale, rows P..2P-1 zero point, row 2P the
// per-slot constant.
#include <type_traits>

#include "common.hpp"

namespace btq {

constexpr int kDqWaves = 4;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Token rows in flight per wave. A row costs NP + kOR loads and about 4
// stores, and the vector-memory counter holds at most 63 operations: with 8
// shards a 4-row ring is the deepest whose waits stay exact.
constexpr int kDqRing = 4;
constexpr int kDqRingSmall = 2;   // the same for short batches (decode): more, shorter waves
// Token rows per sub-step (kSub, a template parameter): the rows consumed,
// staged in LDS and written before the ring refills. 1 when the grid is one
// resident generation (one wave per SIMD): each row's ring slot refills as
// soon as it is consumed, which matters most with nothing else on the SIMD
// to hide the latency. 2 when several waves share a SIMD: half the LDS
// round trips and waits per row.
constexpr int kDqSubMax = 2;
constexpr int64_t kDqGeneration = 1024;   // waves at one per SIMD (256 CUs x 4)
// Chunk stores per lane per row whose LDS reads are issued together: a
// 512-slot tile spans at most 768 features unless over 256 BF16 features
// fall inside it.
constexpr int kStU = 3;

// fp32 -> bf16, round to nearest even: the one rounding of the bf16-output
// receiver. Two values per instruction (v_cvt_pk_bf16_f32): a in the low
// half, b in the high half.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) { return bf16_pair(f, 0.0f) & 0xFFFFu; }

// LDS y row: position i of the row's span (relative to the 16-byte aligned
// feature a4 <= hs) lives at dword cpad(i). Four dwords of padding per 32
// keep each 16-byte chunk contiguous and aligned for the wide reads, and
// spread the lanes' stride-8 scatter over 8 banks per element.
__device__ __forceinline__ uint32_t cpad(uint32_t i) { return i + ((i >> 5) << 2); }

// Dwords per LDS y row for spans of up to `span` features: the padded span
// plus one private dummy dword per lane (idle lanes write there, so no two
// lanes ever store to one address).
__host__ __device__ constexpr int dq_row_dwords(int span) {
  return ((span + 3 + 31) / 32 * 32) * 9 / 8 + kWave;
}

// LDS: 4 waves x kSub y rows of buf_dwords.
// NP: shards. kOR: BF16 registers per row; a tile whose NP*nout BF16 values
// fit in kOR*64 lanes sums them in the ring, a wider tile in a pass after it.
// kR: ring depth. kSub: rows per sub-step. kBf: y is bf16 (one rounding of the fp32 sum) instead of
// fp32.
template <int NP, int kOR, int kR, int kSub, bool kBf>
__global__ __launch_bounds__(256) void decompress_kernel(
    const uint8_t* __restrict__ packed, int pitch, const uint16_t* __restrict__ outl, int64_t T,
    int H, int Hq, int k, int ntiles, int rows_per_wave, int64_t nrowblk, int buf_dwords,
    const float* __restrict__ dec, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cmap, void* __restrict__ y) {
  constexpr uint32_t kYB = kBf ? 2u : 4u;   // bytes per y value
  extern __shared__ __align__(16) char smem[];
  // unit = row block; its blocks of 4 adjacent tiles run on one XCD
  int64_t rb, sub;
  const int ntgrp = (ntiles + kDqWaves - 1) / kDqWaves;
  if (!xcd_unit_block(blockIdx.x, ntgrp, nrowblk, &rb, &sub)) return;
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep
  // everything derived from it (rows, descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = (int)sub * kDqWaves + wave;
  if (c >= ntiles) return;   // past the last tile (no block barrier below)
  const TileGeom g = tile_geom(cmap, c, ntiles, Hq, H);
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min(T - t0, (int64_t)rows_per_wave);   // >= 1
  float* const buf = reinterpret_cast<float*>(smem) + (size_t)wave * kSub * buf_dwords;
  const uint32_t dummy = (uint32_t)(buf_dwords - kWave + lane);

  // Whole message tensors (the launcher checks they span < 2^31 bytes), and
  // this wave's rows of y.
  const rsrc_t rp = make_rsrc(packed, (uint32_t)(NP * T * (int64_t)pitch));
  const rsrc_t ro = make_rsrc(outl, (uint32_t)(NP * T * (int64_t)k * 2));
  const rsrc_t ry = make_rsrc(static_cast<char*>(y) + t0 * H * kYB, (uint32_t)nrows * (uint32_t)H * kYB);
  const rsrc_t rc = make_rsrc(cmap, (uint32_t)Hq * 4u);
  const rsrc_t ri = make_rsrc(idx, (uint32_t)k * 4u);

  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  const uint32_t pk_off = active ? (uint32_t)(j0 >> 1) : kOOB;
  // BF16 block: entry e = r*64 + lane holds shard e / nout, feature e % nout
  const bool compact = NP * g.nout <= kOR * kWave;   // uniform
  uint32_t o_off[kOR];
#pragma unroll
  for (int r = 0; r < kOR; ++r) {
    const int e = r * kWave + lane;
    o_off[r] = kOOB;
    if (g.nout > 0 && compact && e < NP * g.nout) {
      const int sp = e / g.nout, i = e - sp * g.nout;
      o_off[r] = (uint32_t)(((int64_t)sp * T * k + g.ilo + i) * 2);
    }
  }

  uint32_t w[kR][NP], ov[kR][kOR];
  // The lane's offsets stay in fixed VGPRs; the (shard, row) offset is
  // uniform and rides in the instruction's SGPR offset.
  // A row past the wave's last loads out of range. With one wave per SIMD
  // (kSub == 1) through empty descriptors, a scalar choice that spares the
  // per-row selection of every lane offset (7B: 17.6 -> 17.0 us); with
  // several waves per SIMD through the lane offsets, which measured faster
  // there (large prefill 88.8 against 91.8 us).
  auto load = [&](int q, int row) {
    const bool ok = row < nrows;   // uniform
    const int64_t rowg = t0 + min(row, nrows - 1);
    if constexpr (kSub == 1) {
      const rsrc_t rpq = make_rsrc(packed, ok ? (uint32_t)(NP * T * (int64_t)pitch) : 0u);
      const rsrc_t roq = make_rsrc(outl, ok ? (uint32_t)(NP * T * (int64_t)k * 2) : 0u);
#pragma unroll
      for (int p = 0; p < NP; ++p)
        w[q][p] = __builtin_amdgcn_raw_buffer_load_b32(
            rpq, pk_off, (uint32_t)(((int64_t)p * T + rowg) * pitch), kStream);
#pragma unroll
      for (int r = 0; r < kOR; ++r)
        ov[q][r] = __builtin_amdgcn_raw_buffer_load_b16(roq, o_off[r], (uint32_t)(rowg * k * 2),
                                                        0);
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p)
        w[q][p] = __builtin_amdgcn_raw_buffer_load_b32(
            rp, ok ? pk_off : kOOB, (uint32_t)(((int64_t)p * T + rowg) * pitch), kStream);
#pragma unroll
      for (int r = 0; r < kOR; ++r)
        ov[q][r] = __builtin_amdgcn_raw_buffer_load_b16(ro, ok ? o_off[r] : kOOB,
                                                        (uint32_t)(rowg * k * 2), 0);
    }
  };

  // Setup loads first, ring loads second: the vector-memory counter retires
  // in order, so waiting for a setup load never waits for the ring.
  // (a) the lane's 8 slots of every shard's scale row and of the constant
  // row (lanes past the tile read zeros)
  const rsrc_t rd = make_rsrc(dec, (uint32_t)((2 * NP + 1) * (int64_t)Hq * 4));
  const uint32_t d_off = active ? (uint32_t)j0 * 4u : kOOB;
  v4u sv[NP][2], bv[2];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    sv[p][0] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off, (uint32_t)(p * Hq * 4), 0);
    sv[p][1] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off + 16u, (uint32_t)(p * Hq * 4), 0);
  }
  bv[0] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off, (uint32_t)(2 * NP * Hq * 4), 0);
  bv[1] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off + 16u, (uint32_t)(2 * NP * Hq * 4), 0);
  // (b) the lane's 8 feature indices and its BF16 feature index
  const int jj = active ? j0 : g.jstart;
  const v4u hA = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u, 0, 0);
  const v4u hB = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u + 16u, 0, 0);
  const bool own_out = lane < g.nout;
  const uint32_t oh =
      __builtin_amdgcn_raw_buffer_load_b32(ri, own_out ? (uint32_t)(g.ilo + lane) * 4u : kOOB, 0, 0);
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

  // Per-lane constants, settled once (their loads are older than the ring).
  const int a4 = g.hs & ~3;   // first feature of the span's first 16-byte chunk of y
  const int hh[8] = {(int)hA[0], (int)hA[1], (int)hA[2], (int)hA[3],
                     (int)hB[0], (int)hB[1], (int)hB[2], (int)hB[3]};
  float sc[NP][8], bias[8];
  uint32_t ya[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ya[e] = active ? cpad((uint32_t)(hh[e] - a4)) : dummy;
    bias[e] = __uint_as_float(bv[e >> 2][e & 3]);
    settle(bias[e]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float s = __uint_as_float(sv[p][e >> 2][e & 3]);
      sc[p][e] = (e & 1) ? s * 0.0625f : s;   // high nibbles arrive as 16*q
      settle(sc[p][e]);
    }
  }
  // (a lane that owns no BF16 feature reads oh = 0; the clamp keeps its
  // unused address in range, and its write goes to its dummy dword)
  const uint32_t oa = own_out ? cpad((uint32_t)max((int)oh - a4, 0)) : dummy;
  // Lane i < nout owns BF16 feature ilo+i: its shard p value sits in entry
  // p*nout + i, i.e. register (entry / 64) of lane (entry % 64).
  int src_addr[NP], src_reg[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e = p * g.nout + (own_out ? lane : 0);
    src_addr[p] = (e & (kWave - 1)) * 4;
    src_reg[p] = min(e >> 6, kOR - 1);
  }
  const int nreg = (NP * g.nout + kWave - 1) / kWave;   // BF16 registers this tile uses
  // y stores: whole 16-byte chunks q_lo..q_hi-1 of the span, plus at most 3
  // ragged features at each end (lanes 0-2 and 3-5), one dword each.
  const int q_lo = (g.hs - a4 + 3) >> 2;
  const int q_hi = max((g.he - a4) >> 2, q_lo);
  const int st_it = (q_hi - q_lo + kWave - 1) / kWave;   // uniform
  int bpos = -1;
  if (lane < 3) {
    const int h = g.hs + lane;
    if (h < min(a4 + 4 * q_lo, g.he)) bpos = h;
  } else if (lane < 6) {
    const int h = a4 + 4 * q_hi + (lane - 3);
    if (h < g.he) bpos = h;
  }
  const uint32_t b_lds = cpad((uint32_t)(max(bpos, g.hs) - a4));
  const uint32_t b_off = bpos >= 0 ? (uint32_t)bpos * kYB : kOOB;

  // y stores of one 16-byte chunk (4 features) and of one feature. The
  // chunk store reaches its row through a per-row descriptor and takes an
  // immediate zero as its scalar offset. A store wider than 64 bits reads
  // its data registers after issue, so a VALU write to them on the next
  // instruction needs one wait state. The compiler inserts it only for an
  // immediate scalar offset: with a register there it lets the next
  // instruction overwrite the data, and on gfx950 the stored values then
  // come out wrong.
  char* const ybase = static_cast<char*>(y) + t0 * H * kYB;
  // (a row past the wave's last stores through an empty descriptor, so the
  // lanes' offsets are the same for every row)
  auto row_rsrc = [&](int row) {
    return make_rsrc(ybase + (int64_t)min(row, nrows - 1) * H * kYB,
                     row < nrows ? (uint32_t)H * kYB : 0u);
  };
  auto store_chunk = [&](const v4f& v, uint32_t off, const rsrc_t& rr) {
    if constexpr (kBf) {
      typedef unsigned int v2u __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(v2u{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3])}, rr,
                                            off, 0, kStream);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(
          v4u{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
              __float_as_uint(v[3])},
          rr, off, 0, kStream);
    }
  };
  auto store_one = [&](float f, uint32_t off, const rsrc_t& rr) {
    if constexpr (kBf)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bf16_bits_rne(f), rr, off, 0, kStream);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), rr, off, 0, kStream);
  };
  // the lane's chunk offsets for the usual spans (out of range past the span)
  uint32_t c_off[kStU];
#pragma unroll
  for (int it = 0; it < kStU; ++it) {
    const int qc = q_lo + lane + kWave * it;
    c_off[it] = qc < q_hi ? (uint32_t)(a4 + 4 * qc) * kYB : kOOB;
  }

  // nrows >= 1: a do-while has no entry guard that the ring loads could be
  // sunk below.
  int base = 0;
  do {
#pragma unroll
    for (int sb = 0; sb < kR / kSub; ++sb) {
#pragma unroll
      for (int r = 0; r < kSub; ++r) {
        const int q = sb * kSub + r;
        float* b = buf + r * buf_dwords;
        // BF16 values first: the cross-lane reads are issued before the
        // dequantization, so their LDS round trip overlaps it. Only the
        // registers the tile fills are read (nreg is uniform); the others
        // are never selected below.
        const bool bf_row = compact && g.nout > 0;   // uniform
        int t[NP][kOR];
        if (bf_row) {
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            t[p][0] = __builtin_amdgcn_ds_bpermute(src_addr[p], (int)(ov[q][0] << 16));
#pragma unroll
            for (int rr = 1; rr < kOR; ++rr) t[p][rr] = 0;
          }
          if (nreg > 1) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
#pragma unroll
              for (int rr = 1; rr < kOR; ++rr)
                t[p][rr] = __builtin_amdgcn_ds_bpermute(src_addr[p], (int)(ov[q][rr] << 16));
            }
          }
        }
        issue_fence();
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          uint32_t lo = w[q][p] & 0x0F0F0F0Fu;
          uint32_t hi = w[q][p] & 0xF0F0F0F0u;
          // Opaque to the optimizer: otherwise it folds each mask into a
          // per-byte extract, one more instruction per code. Kept whole, each
          // byte converts directly (v_cvt_f32_ubyte0..3).
          opaque(lo);
          opaque(hi);
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            acc[2 * bb] = fmaf((float)((lo >> (8 * bb)) & 0xFFu), sc[p][2 * bb], acc[2 * bb]);
            acc[2 * bb + 1] =
                fmaf((float)((hi >> (8 * bb)) & 0xFFu), sc[p][2 * bb + 1], acc[2 * bb + 1]);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) b[ya[e]] = acc[e];
        if (bf_row) {
          // the owner lane's shard values, added in shard order from 0
          float o = 0.0f;
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            int v = t[p][0];
#pragma unroll
            for (int rr = 1; rr < kOR; ++rr) v = (src_reg[p] == rr) ? t[p][rr] : v;
            // (each value was moved to the high half before the cross-lane
            // read: its fp32 bits)
            o = __fadd_rn(o, __uint_as_float((uint32_t)v));
          }
          b[oa] = o;
        }
      }
      // refill the consumed slots with the rows kR ahead
#pragma unroll
      for (int r = 0; r < kSub; ++r) load(sb * kSub + r, base + kR + sb * kSub + r);
      wave_lds_sync();
      if (st_it <= kStU) {   // uniform: the usual case
        // Every LDS read of the sub-step is issued before its first store,
        // so one LDS round trip is exposed per sub-step, not one per chunk.
        // (a chunk index past the span is clamped into it; its lane's store
        // is out of range)
        v4f cv[kSub][kStU];
        float rv[kSub];
#pragma unroll
        for (int r = 0; r < kSub; ++r) {
          const float* b = buf + r * buf_dwords;
#pragma unroll
          for (int it = 0; it < kStU; ++it) {
            const int qc = min(q_lo + lane + kWave * it, q_hi - 1);
            cv[r][it] = *reinterpret_cast<const v4f*>(b + cpad((uint32_t)(4 * max(qc, 0))));
          }
          rv[r] = b[b_lds];
        }
#pragma unroll
        for (int r = 0; r < kSub; ++r) {
          const rsrc_t rr = row_rsrc(base + sb * kSub + r);
#pragma unroll
          for (int it = 0; it < kStU; ++it) store_chunk(cv[r][it], c_off[it], rr);
          store_one(rv[r], b_off, rr);
        }
      } else {
#pragma unroll
        for (int r = 0; r < kSub; ++r) {
          const float* b = buf + r * buf_dwords;
          const rsrc_t rr = row_rsrc(base + sb * kSub + r);
          for (int it = 0; it < st_it; ++it) {
            const int qc = q_lo + lane + kWave * it;
            const v4f v = *reinterpret_cast<const v4f*>(b + cpad((uint32_t)(4 * min(qc, q_hi - 1))));
            store_chunk(v, qc < q_hi ? (uint32_t)(a4 + 4 * qc) * kYB : kOOB, rr);
          }
          store_one(b[b_lds], b_off, rr);
        }
      }
      wave_lds_sync();
    }
    base += kR;
  } while (base < nrows);

  if (!compact) {   // uniform
    // More BF16 values than the ring's registers hold: the loop stored stale
    // LDS values at these features. Wait until those stores are complete, then
    // write the sums over the shards, in shard order from 0.
    __builtin_amdgcn_s_waitcnt(0);
    // 4 entries per lane per trip, all their loads in flight together
    constexpr int kPer = 4;
    const int n = nrows * g.nout;
    for (int e0 = 0; e0 < n; e0 += kPer * kWave) {
      uint32_t hv[kPer], v[kPer][NP], yo[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int eu = e0 + u * kWave + lane;
        const int e = min(eu, n - 1);
        const int r = e / g.nout, i = e - r * g.nout;
        hv[u] = __builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)(g.ilo + i) * 4u, 0, 0);
        yo[u] = eu < n ? (uint32_t)r * (uint32_t)H * kYB : kOOB;
#pragma unroll
        for (int p = 0; p < NP; ++p)
          v[u][p] = __builtin_amdgcn_raw_buffer_load_b16(
              ro, (uint32_t)(((int64_t)p * T * k + g.ilo + i) * 2), (uint32_t)((t0 + r) * k * 2), 0);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        float o = 0.0f;
#pragma unroll
        for (int p = 0; p < NP; ++p) o = __fadd_rn(o, bf16_to_f32(v[u][p]));
        // (an entry past the end stores out of range)
        const uint32_t off = yo[u] == kOOB ? kOOB : yo[u] + hv[u] * kYB;
        if constexpr (kBf)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bf16_bits_rne(o), ry, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ry, off, 0, 0);
      }
    }
  }
}

template <bool kBf>
__global__ __launch_bounds__(256) void decompress_general_kernel(
    const uint8_t* __restrict__ packed, int64_t pitch, const uint16_t* __restrict__ outl, int64_t P,
    int64_t T, int64_t H, int64_t k, int64_t Hq, const float* __restrict__ dec,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap, void* __restrict__ y) {
  auto put = [&](int64_t i, float v) {
    if constexpr (kBf)
      static_cast<uint16_t*>(y)[i] = (uint16_t)bf16_bits_rne(v);
    else
      static_cast<float*>(y)[i] = v;
  };
  const int64_t n1 = T * Hq;
  const int64_t n2 = T * k;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1 + n2; i += stride) {
    float acc = 0.0f;
    if (i < n1) {
      const int64_t t = i / Hq, j = i % Hq;
      const int64_t h = cmap[j];
      for (int64_t p = 0; p < P; ++p) {
        const uint32_t byte = packed[(p * T + t) * pitch + (j >> 1)];
        const int q = (int)((j & 1) ? (byte >> 4) : (byte & 0xFu));
        const float d = __fsub_rn((float)q, dec[(P + p) * Hq + j]);   // exact
        acc = __fadd_rn(acc, __fmul_rn(d, dec[p * Hq + j]));
      }
      put(t * H + h, acc);
    } else {
      const int64_t ii = i - n1;
      const int64_t t = ii / k, o = ii % k;
      for (int64_t p = 0; p < P; ++p) acc = __fadd_rn(acc, bf16_to_f32(outl[(p * T + t) * k + o]));
      put(t * H + idx[o], acc);
    }
  }
}

template <int NP, int kOR, int kR, int kSub, bool kBf>
static void launch_fast(const uint8_t* packed, int64_t pitch, const uint16_t* outl, int64_t T,
                        int64_t H,
                        int64_t k, int64_t Hq, int ntiles, int rpw, int64_t nrowblk,
                        int buf_dwords, const float* dec, const int32_t* idx,
                        const int32_t* cmap, void* y, hipStream_t s) {
  const int64_t ntgrp = (ntiles + kDqWaves - 1) / kDqWaves;
  const size_t lds = (size_t)kDqWaves * kSub * buf_dwords * 4;
  decompress_kernel<NP, kOR, kR, kSub, kBf><<<(unsigned)xcd_grid(ntgrp, nrowblk), 256, lds, s>>>(
      packed, (int)pitch, outl, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, buf_dwords, dec,
      idx, cmap, y);
}

template <bool kBf>
static void dispatch_fast(int64_t P, bool wide, bool small, bool one_gen, const uint8_t* packed,
                          int64_t pitch, const uint16_t* outl, int64_t T, int64_t H, int64_t k,
                          int64_t Hq, int ntiles, int rpw, int64_t nrowblk, int buf_dwords,
                          const float* dec, const int32_t* idx, const int32_t* cmap, void* y,
                          hipStream_t s) {
  // (the 2-row ring serves short batches, whose grids are one generation)
  switch (P) {
#define BTQ_DQ_ARGS \
  packed, pitch, outl, T, H, k, Hq, ntiles, rpw, nrowblk, buf_dwords, dec, idx, cmap, y, s
#define BTQ_DQ_CASE(n)                                                        \
  case n:                                                                     \
    if (wide && small)                                                        \
      launch_fast<n, 4, kDqRingSmall, 1, kBf>(BTQ_DQ_ARGS);                   \
    else if (wide && one_gen)                                                 \
      launch_fast<n, 4, kDqRing, 1, kBf>(BTQ_DQ_ARGS);                        \
    else if (wide)                                                            \
      launch_fast<n, 4, kDqRing, 2, kBf>(BTQ_DQ_ARGS);                        \
    else if (small)                                                           \
      launch_fast<n, 2, kDqRingSmall, 1, kBf>(BTQ_DQ_ARGS);                   \
    else if (one_gen)                                                         \
      launch_fast<n, 2, kDqRing, 1, kBf>(BTQ_DQ_ARGS);                        \
    else                                                                      \
      launch_fast<n, 2, kDqRing, 2, kBf>(BTQ_DQ_ARGS);                        \
    break;
    BTQ_DQ_CASE(1)
    BTQ_DQ_CASE(2)
    BTQ_DQ_CASE(3)
    BTQ_DQ_CASE(4)
    BTQ_DQ_CASE(5)
    BTQ_DQ_CASE(6)
    BTQ_DQ_CASE(7)
    BTQ_DQ_CASE(8)
#undef BTQ_DQ_CASE
#undef BTQ_DQ_ARGS
  }
}

hipError_t launch_decompress(const uint8_t* packed, int64_t pitch, const uint16_t* outl, int64_t P,
                             int64_t T, int64_t H, int64_t k, const float* dec, const int32_t* idx,
                             const int32_t* cmap, void* y, bool bf16, hipStream_t s) {
  const int64_t yb = bf16 ? 2 : 4;   // bytes per y value
  const int64_t Hq = H - k;
  const int64_t span = (H < kTileSlots + k ? H : kTileSlots + k);
  const int buf_dwords = span < 65536 ? dq_row_dwords((int)span) : (1 << 30);
  // (LDS for the larger sub-step, whichever the launch takes)
  const size_t lds = (size_t)kDqWaves * kDqSubMax * buf_dwords * 4;
  // Buffer resources: the whole message, the decoder table and one wave's
  // rows of y must each span fewer than 2^31 bytes. y rows take stores of 4
  // values (16 bytes fp32, 8 bytes bf16): H a multiple of 4 and y aligned to
  // one such store.
  const int64_t lim = int64_t(1) << 31;
  const bool fast = Hq > 0 && P <= 8 && Hq % 8 == 0 && H % 4 == 0 &&
                    (uintptr_t)packed % 4 == 0 && (uintptr_t)dec % 16 == 0 &&
                    (uintptr_t)y % (4 * yb) == 0 && lds <= 65536 && pitch % 4 == 0 &&
                    P * T * pitch < lim &&
                    P * T * k * 2 < lim && (2 * P + 1) * Hq * 4 < lim && 64 * H * yb < lim;
  if (fast) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    // about 1024 waves (4 per CU: each wave's table loads then serve at
    // least 16 rows where the batch allows), a multiple of the ring depth,
    // up to 64 rows; batches too short to give every wave a full 8-row ring
    // take the 2-row ring. The bf16-output receiver writes half the bytes
    // and gains from two waves per SIMD once the batch has 32768 row-tiles
    // or more (about 2048 waves): 7B at T=8192 51.6 -> 47.2 us, large prefill
    // at T=4096 36.3 -> 32.3 us; the fp32 receiver loses there (7B at
    // T=8192 56.2 -> 59.5 us).
    const int64_t waves = (bf16 && ntiles * T >= 32768) ? 2 * kDqGeneration : kDqGeneration;
    int64_t rpw64 = (ntiles * T + waves - 1) / waves;
    const bool small = rpw64 < kDqRing;
    const int ring = small ? kDqRingSmall : kDqRing;
    rpw64 = (rpw64 + ring - 1) / ring * ring;
    if (rpw64 < ring) rpw64 = ring;
    if (rpw64 > 64) rpw64 = 64;
    const int rpw = (int)rpw64;
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    // BF16 registers per row: 2 (128 shard x feature values per tile) while a
    // tile holds at most 64 of them on average, else 4. A tile beyond its
    // registers sums its BF16 features after the row loop.
    const bool wide = P * k > int64_t(kWave) * ntiles;
    // one sub-step row while the grid is one generation (at most one wave per
    // SIMD), two once several waves share each SIMD
    const bool one_gen = ntiles * nrowblk <= kDqGeneration;
    if (bf16)
      dispatch_fast<true>(P, wide, small, one_gen, packed, pitch, outl, T, H, k, Hq, ntiles, rpw,
                          nrowblk, buf_dwords, dec, idx, cmap, y, s);
    else
      dispatch_fast<false>(P, wide, small, one_gen, packed, pitch, outl, T, H, k, Hq, ntiles, rpw,
                           nrowblk, buf_dwords, dec, idx, cmap, y, s);
    return hipGetLastError();
  }
  const int64_t n = T * H;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (bf16)
    decompress_general_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(packed, pitch, outl, P, T, H,
                                                                     k, Hq, dec, idx, cmap, y);
  else
    decompress_general_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(packed, pitch, outl, P, T, H,
                                                                      k, Hq, dec, idx, cmap, y);
  return hipGetLastError();
}

}  // namespace btq
