// HIP kernels for gfx950 (CDNA4): slot-mapped KV append, paged decode
// attention, and the split-K log-sum-exp combine.
//
// Method: one query token per sequence attends to its cached tokens, which
// live in fixed-size physical blocks reached through a per-sequence block
// table; the per-block softmax is accumulated online (running max and sum,
// rescaled when the max grows) and, for long contexts, partitions of the
// context produce partial results that a reduce step combines
// ("PagedAttention from First Principles", sections 5 and 17; Equation 4 of
// the hungchun0201 vLLM digest).  The pages' kernel sketch (one warp per block,
// reduce across warps) targets other hardware; the design here is gfx950's:
//
// * Work unit = (kv head [x column group], sequence, partition of the
//   context); a workgroup of 4 wave64s, each wave walking every 4th 16-token
//   tile of the partition with the next two tiles' loads in flight while it
//   computes on the current one.
// * Pool layouts (K [NB, Hkv, D/8, B, 8], V [NB, Hkv, B/4, D, 4]) make every
//   16-byte lane load land directly in MFMA operand order, 256 contiguous
//   bytes per 16 lanes, so there is no LDS staging of K/V and no shuffles
//   before the matrix cores.  Tiles are read with buffer loads whose resource
//   descriptor is built per tile in scalar registers from the block-table
//   entry; a descriptor with zero records turns the pipeline's padding loads
//   past a wave's last tile into free zero loads, so the loop never branches
//   around a load.
// * GQA path (q heads per KV head >= 3): QK^T is v_mfma_f32_16x16x32_bf16 with
//   16 tokens as rows and the group's query heads as columns; PV is
//   v_mfma_f32_16x16x16_bf16 whose B operand is exactly the QK^T accumulator
//   layout, so probabilities go from scores to PV without moving between
//   lanes.  P is split into a high and a low bf16 part (two MFMAs) so the PV
//   product keeps ~16 significant bits of P.
// * MHA path (1 or 2 q heads per KV head): fp32 FMAs on the same loads,
//   cross-lane sums with wave shuffles.
// * The softmax reference max is raised lazily: only when a tile's max
//   exceeds it by more than 2^8 in probability, so the accumulator rescale
//   runs on a handful of tiles instead of every tile.  Results are the same
//   quantity (numerator and denominator share the reference).
// * Split contexts: each partition writes (reference max, sum, normalised
//   output) to a workspace; a second kernel combines the partitions of every
//   (sequence, head) in ascending order (deterministic).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_internal.h"

namespace pa {

WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                                 int64_t max_parts) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WorkspaceLayout w;
  w.ml_off = 0;
  w.o_off = up(sizeof(float) * 2 * size_t(num_seqs * num_q_heads * max_parts));
  w.total = w.o_off + up(sizeof(float) * size_t(num_seqs * num_q_heads * max_parts * head_dim));
  return w;
}

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();
// gfx9 buffer descriptor word 3 for raw dword access
constexpr int kBufferFlags = 0x00020000;
// a byte offset no tile reaches: buffer loads at it return zeros, touching no memory
constexpr uint32_t kOutOfRange = 0x80000000u;
// lazy rescale threshold (log2 units): probabilities stay <= 2^8
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// bf16 pair -> two floats (exact)
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, kBufferFlags);
}

// K/V tiles are read once per decode step: non-temporal loads (the nt bit)
// stream them without displacing cached data, and on MI355X sustain ~25 %
// more HBM read bandwidth than default-policy loads for 4 KiB random tiles.
constexpr int kStreamingLoad = 2;

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kStreamingLoad));
}

// ---------------------------------------------------------------------------
// tile addressing
//
// A tile is 16 consecutive tokens of one KV head.  Lane l holds
//   K: token row r = l & 15, for chunk c the dims 8*((l >> 4) + 4c) .. +7;
//   V: tokens 4*(l >> 4) .. +3, for chunk c the dims 2*(l & 15) + 32c and +1;
// one 16-byte load per chunk each, D/32 chunks.  The byte offsets of a lane
// inside its block tile are fixed for the kernel.
// ---------------------------------------------------------------------------
template <int D, int BS>
struct LaneOffsets {
  uint32_t k0, k1, v0, v1;  // byte offsets; k1/v1 used for the second block of a B = 8 tile
};

template <int D, int BS>
__device__ __forceinline__ LaneOffsets<D, BS> lane_offsets(int lane) {
  const int r = lane & 15;
  const int g4 = lane >> 4;
  LaneOffsets<D, BS> o;
  if constexpr (BS == 8) {
    // rows 0-7 and token quads 0-1 come from the first block, the rest from the second
    const uint32_t k = uint32_t((g4 * BS + (r & 7)) * 8 * 2);
    const uint32_t v = uint32_t(((g4 & 1) * D + 2 * r) * 4 * 2);
    o.k0 = (r >> 3) ? kOutOfRange : k;
    o.k1 = (r >> 3) ? k : kOutOfRange;
    o.v0 = (g4 >> 1) ? kOutOfRange : v;
    o.v1 = (g4 >> 1) ? v : kOutOfRange;
  } else {
    o.k0 = uint32_t((g4 * BS + r) * 8 * 2);
    o.v0 = uint32_t((g4 * D + 2 * r) * 4 * 2);
    o.k1 = o.v1 = 0;
  }
  return o;
}

// Load tile `ts` (wave-uniform first token) whose physical block(s) are
// phys0 / phys1, or zeros without any memory access when !valid.
template <int D, int BS>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int kvh, int phys0, int phys1,
                                          int ts, bool valid, const LaneOffsets<D, BS>& lo,
                                          u32x4 (&k)[D / 32], u32x4 (&v)[D / 32]) {
  constexpr int kTileBytes = BS * D * 2;
  const size_t blk_elems = size_t(p.num_kv_heads) * BS * D;
  const size_t head_off = size_t(kvh) * BS * D;
  const int bytes = valid ? kTileBytes : 0;
  const __amdgpu_buffer_rsrc_t k0 = tile_rsrc(p.k_cache + size_t(phys0) * blk_elems + head_off, bytes);
  const __amdgpu_buffer_rsrc_t v0 = tile_rsrc(p.v_cache + size_t(phys0) * blk_elems + head_off, bytes);
  if constexpr (BS == 8) {
    const __amdgpu_buffer_rsrc_t k1 = tile_rsrc(p.k_cache + size_t(phys1) * blk_elems + head_off, bytes);
    const __amdgpu_buffer_rsrc_t v1 = tile_rsrc(p.v_cache + size_t(phys1) * blk_elems + head_off, bytes);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      k[c] = buffer_load16(k0, lo.k0 + c * 4 * BS * 16) | buffer_load16(k1, lo.k1 + c * 4 * BS * 16);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      v[c] = buffer_load16(v0, lo.v0 + c * 256) | buffer_load16(v1, lo.v1 + c * 256);
  } else {
    // B = 32 holds two tiles per block: the second half starts 16 tokens in
    const uint32_t khalf = BS == 32 ? uint32_t(((ts >> 4) & 1) * 16 * 8 * 2) : 0u;
    const uint32_t vhalf = BS == 32 ? uint32_t(((ts >> 4) & 1) * 4 * D * 4 * 2) : 0u;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) k[c] = buffer_load16(k0, lo.k0 + khalf + c * 4 * BS * 16);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) v[c] = buffer_load16(v0, lo.v0 + vhalf + c * 256);
  }
  // keep the scheduler from hoisting the previous tile's math above these
  // loads: issuing them first is what keeps bytes in flight
  __builtin_amdgcn_sched_barrier(0);
}

// Block-table entries of up to 64 consecutive tiles of one wave, one per lane,
// so the tile loop never waits on memory for an address: lane j holds the
// physical block of the wave's tile k0 + j (b1: second block when B = 8;
// the first block again when that half lies past the context).
struct TableCache {
  int b0, b1;
};

template <int BS>
__device__ __forceinline__ TableCache fetch_table(const int32_t* bt, int t0, int t1, int wave,
                                                  int k0, int n, int lane) {
  TableCache c{0, 0};
  const int k = k0 + lane;
  if (k < n) {
    const int ts = t0 + 16 * (wave + kWaves * k);
    if constexpr (BS == 16) {
      c.b0 = bt[ts >> 4];
    } else if constexpr (BS == 32) {
      c.b0 = bt[ts >> 5];
    } else {
      c.b0 = bt[ts >> 3];
      c.b1 = (ts + 8 < t1) ? bt[(ts >> 3) + 1] : c.b0;
    }
  }
  return c;
}

// Walk this wave's tiles (tiles wave, wave + 4, ... of the partition [t0, t1))
// with the next two tiles' loads issued before the current tile is computed.
// Every compute is preceded by the same number of younger loads on every path
// (past the last tile the loads are zero-record no-ops), so the compiler waits
// only for the tile it is about to use.
template <int D, int BS, typename F>
__device__ __forceinline__ void walk_tiles(const DecodeParams& p, const int32_t* bt, int kvh,
                                           int t0, int t1, int wave, int lane, F&& compute) {
  constexpr int NC = D / 32;
  const int ntiles = (t1 - t0 + 15) >> 4;
  const int n = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const LaneOffsets<D, BS> lo = lane_offsets<D, BS>(lane);
  for (int k0 = 0; k0 < n; k0 += 64) {
    const TableCache tc = fetch_table<BS>(bt, t0, t1, wave, k0, n, lane);
    const int m = min(64, n - k0);
    auto start = [&](int j) { return t0 + 16 * (wave + kWaves * (k0 + j)); };
    auto load = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
      const int jj = min(j, m - 1);
      const int b0 = __builtin_amdgcn_readlane(tc.b0, jj);
      const int b1 = BS == 8 ? __builtin_amdgcn_readlane(tc.b1, jj) : 0;
      load_tile<D, BS>(p, kvh, b0, b1, start(jj), j < m, lo, kt, vt);
    };
    u32x4 ak[NC], av[NC], bk[NC], bv[NC], ck[NC], cv[NC];
    load(0, ak, av);
    load(1, bk, bv);
    for (int j = 0;; j += 3) {
      load(j + 2, ck, cv);
      compute(start(j), ak, av);
      if (j + 1 >= m) break;
      load(j + 3, ak, av);
      compute(start(j + 1), bk, bv);
      if (j + 2 >= m) break;
      load(j + 4, bk, bv);
      compute(start(j + 2), ck, cv);
      if (j + 3 >= m) break;
    }
  }
}

// Zero the V values of tokens at or past t1 (0 * NaN would poison the sum).
// Branch-free: on full tiles the masks are all ones.
template <int D>
__device__ __forceinline__ void mask_v(u32x4 (&v)[D / 32], int ts, int t1, int lane) {
  const int tq = ts + 4 * (lane >> 4);
  const uint32_t m01 = (tq + 0 < t1 ? 0x0000ffffu : 0u) | (tq + 1 < t1 ? 0xffff0000u : 0u);
  const uint32_t m23 = (tq + 2 < t1 ? 0x0000ffffu : 0u) | (tq + 3 < t1 ? 0xffff0000u : 0u);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    v[c].x &= m01;
    v[c].y &= m23;
    v[c].z &= m01;
    v[c].w &= m23;
  }
}

// Per-workgroup LDS for the cross-wave combine.
template <int D>
struct Smem {
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][D][17];
};

__device__ __forceinline__ void store_out(const DecodeParams& p, int s, int h, int d, float r) {
  const size_t at = size_t(s) * p.out_s + size_t(h) * p.out_h + d;
  if (p.out_f32)
    static_cast<float*>(p.out)[at] = r;
  else
    static_cast<uint16_t*>(p.out)[at] = uint16_t(bf16_bits(r));
}

// Combine the waves' (m, l, o) and write either the output (one partition)
// or this partition's partial result for the combine kernel.
template <int D>
__device__ __forceinline__ void finish(const DecodeParams& p, Smem<D>& sm, int s, int h0, int ncols,
                                       int part, int nparts) {
  __syncthreads();
  for (int idx = threadIdx.x; idx < ncols * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][g]);
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float e = exp2f(sm.m[w][g] - M);
        o += sm.o[w][d][g] * e;
        l += sm.l[w][g] * e;
      }
    }
    const int h = h0 + g;
    if (nparts <= 1) {
      store_out(p, s, h, d, l > 0.f ? o / l : 0.f);
    } else {
      const size_t row = (size_t(s) * p.num_q_heads + h) * p.max_parts + part;
      p.ws_o[row * D + d] = o / l;
      if (d == 0) {
        p.ws_ml[row * 2 + 0] = M;
        p.ws_ml[row * 2 + 1] = l;
      }
    }
  }
}

// Partitions of sequence s that this launch covers (contexts longer than the
// launch covers violate the caller's contract; clamping keeps the partition
// count consistent with the grid).
__device__ __forceinline__ int partitions(const DecodeParams& p, int L) {
  return min((L + p.part_tokens - 1) / p.part_tokens, p.max_parts);
}

// ---------------------------------------------------------------------------
// GQA decode on the matrix cores
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_mfma(DecodeParams p) {
  constexpr int NC = D / 32;  // 16-byte chunks per lane per tile, for K and for V
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int hg = blockIdx.x;
  const int kvh = hg / p.head_groups;
  const int cgrp = hg - kvh * p.head_groups;
  const int s = blockIdx.y;
  const int part = blockIdx.z;

  const int L = p.context_lens[s];
  const int nparts = partitions(p, L);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int t0 = part * p.part_tokens;
  const int t1 = min(L, t0 + p.part_tokens);
  const int h0 = kvh * p.group + cgrp * 16;
  const int ncols = min(16, p.group - cgrp * 16);
  const int32_t* bt = p.block_tables + size_t(s) * p.bt_s;

  // Q as the B operand of QK^T: column r = query head h0 + r (zero past the group)
  u32x4 qv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qv[c] = u32x4{0u, 0u, 0u, 0u};
    if (r < ncols) qv[c] = load16(p.q + size_t(s) * p.q_s + size_t(h0 + r) * p.q_h + 8 * (g4 + 4 * c));
  }

  f32x4 oacc[2 * NC];
#pragma unroll
  for (int i = 0; i < 2 * NC; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;  // reference max (log2 units) of column r
  float l_run = 0.f;      // this lane's share of the running sum of column r

  auto compute = [&](int ts, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) sacc = mfma_16x16x32(kt[c], qv[c], sacc);
    // lane holds scores of tokens ts + 4*g4 + j for query head column r
    float sc[4];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = (ts + 4 * g4 + j < t1) ? sacc[j] * p.scale_log2 : kNegInf;
      mt = fmaxf(mt, sc[j]);
    }
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    if (__any(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 2 * NC; ++i) oacc[i] *= alpha;
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[j] = exp2f(sc[j] - m_run);
      l_run += pr[j];
    }
    // P as the B operand of PV, split into hi + lo bf16
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hb[j] = bf16_bits(pr[j]);
      lb[j] = bf16_bits(pr[j] - bf16_value(hb[j]));
    }
    const u32x2 phi = {hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    const u32x2 plo = {lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
    mask_v<D>(vt, ts, t1, lane);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x2 a0 = {vt[c].x, vt[c].y};  // dim 2r + 32c, tokens 4*g4 .. +3
      const u32x2 a1 = {vt[c].z, vt[c].w};  // dim 2r + 32c + 1
      oacc[2 * c] = mfma_16x16x16(a0, phi, oacc[2 * c]);
      oacc[2 * c] = mfma_16x16x16(a0, plo, oacc[2 * c]);
      oacc[2 * c + 1] = mfma_16x16x16(a1, phi, oacc[2 * c + 1]);
      oacc[2 * c + 1] = mfma_16x16x16(a1, plo, oacc[2 * c + 1]);
    }
  };

  walk_tiles<D, BS>(p, bt, kvh, t0, t1, wave, lane, compute);

  // column totals over the four 16-lane groups
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  if (g4 == 0) {
    sm.m[wave][r] = m_run;
    sm.l[wave][r] = l_run;
  }
#pragma unroll
  for (int mm = 0; mm < 2 * NC; ++mm)
#pragma unroll
    for (int j = 0; j < 4; ++j) sm.o[wave][2 * (4 * g4 + j) + 32 * (mm >> 1) + (mm & 1)][r] = oacc[mm][j];

  finish<D>(p, sm, s, h0, ncols, part, nparts);
}

// ---------------------------------------------------------------------------
// MHA decode (1 or 2 query heads per KV head) on the vector ALUs
// ---------------------------------------------------------------------------
template <int D, int BS, int VG>
__global__ __launch_bounds__(kThreads) void decode_valu(DecodeParams p) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int part = blockIdx.z;

  const int L = p.context_lens[s];
  const int nparts = partitions(p, L);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int t0 = part * p.part_tokens;
  const int t1 = min(L, t0 + p.part_tokens);
  const int h0 = kvh * VG;
  const int32_t* bt = p.block_tables + size_t(s) * p.bt_s;

  // this lane's q dims: 8*(g4 + 4c) + e
  float qf[VG][NC][8];
#pragma unroll
  for (int g = 0; g < VG; ++g)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 u = load16(p.q + size_t(s) * p.q_s + size_t(h0 + g) * p.q_h + 8 * (g4 + 4 * c));
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[g][c][2 * e] = bf_lo(w[e]);
        qf[g][c][2 * e + 1] = bf_hi(w[e]);
      }
    }

  float o[VG][NC][2];
  float m_run[VG], l_run[VG];
#pragma unroll
  for (int g = 0; g < VG; ++g) {
    m_run[g] = kNegInf;
    l_run[g] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[g][c][0] = o[g][c][1] = 0.f;
  }

  auto compute = [&](int ts, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    float kf[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t w[4] = {kt[c].x, kt[c].y, kt[c].z, kt[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[c][2 * e] = bf_lo(w[e]);
        kf[c][2 * e + 1] = bf_hi(w[e]);
      }
    }
    mask_v<D>(vt, ts, t1, lane);
    const bool valid = ts + r < t1;
#pragma unroll
    for (int g = 0; g < VG; ++g) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(kf[c][e], qf[g][c][e], dot);
      dot += shfl_xor(dot, 16);
      dot += shfl_xor(dot, 32);
      const float sc = valid ? dot * p.scale_log2 : kNegInf;  // score of token ts + r
      float mt = sc;
      mt = fmaxf(mt, shfl_xor(mt, 1));
      mt = fmaxf(mt, shfl_xor(mt, 2));
      mt = fmaxf(mt, shfl_xor(mt, 4));
      mt = fmaxf(mt, shfl_xor(mt, 8));
      float alpha = 1.f;
      if (mt > m_run[g] + kRescaleSlack) {  // uniform: mt and m_run are the same in every lane
        const float m_new = fmaxf(m_run[g], mt);
        alpha = exp2f(m_run[g] - m_new);
        l_run[g] *= alpha;
        m_run[g] = m_new;
      }
      const float pr = exp2f(sc - m_run[g]);
      l_run[g] += pr;
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = __shfl(pr, 4 * g4 + j, 64);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float a0 = o[g][c][0] * alpha, a1 = o[g][c][1] * alpha;
        a0 = fmaf(pj[0], bf_lo(vt[c].x), a0);
        a0 = fmaf(pj[1], bf_hi(vt[c].x), a0);
        a0 = fmaf(pj[2], bf_lo(vt[c].y), a0);
        a0 = fmaf(pj[3], bf_hi(vt[c].y), a0);
        a1 = fmaf(pj[0], bf_lo(vt[c].z), a1);
        a1 = fmaf(pj[1], bf_hi(vt[c].z), a1);
        a1 = fmaf(pj[2], bf_lo(vt[c].w), a1);
        a1 = fmaf(pj[3], bf_hi(vt[c].w), a1);
        o[g][c][0] = a0;
        o[g][c][1] = a1;
      }
    }
  };

  walk_tiles<D, BS>(p, bt, kvh, t0, t1, wave, lane, compute);

#pragma unroll
  for (int g = 0; g < VG; ++g) {
    float l = l_run[g];  // per-token shares: sum over the 16 token lanes
    l += shfl_xor(l, 1);
    l += shfl_xor(l, 2);
    l += shfl_xor(l, 4);
    l += shfl_xor(l, 8);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float x = o[g][c][e];  // per-quad shares: sum over the four 16-lane groups
        x += shfl_xor(x, 16);
        x += shfl_xor(x, 32);
        if (g4 == 0) sm.o[wave][2 * r + 32 * c + e][g] = x;
      }
    if (lane == 0) {
      sm.m[wave][g] = m_run[g];
      sm.l[wave][g] = l;
    }
  }

  finish<D>(p, sm, s, h0, VG, part, nparts);
}

// ---------------------------------------------------------------------------
// split-K combine: out = sum_p w_p o_p / sum_p w_p with w_p = l_p 2^(m_p - M),
// M = max_p m_p, partitions in ascending order.  One thread per (head, dim).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
  const int s = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.num_q_heads * D) return;
  const int nparts = partitions(p, p.context_lens[s]);
  if (nparts <= 1) return;  // the decode kernel wrote this row directly
  const int h = idx / D;
  const int d = idx - h * D;
  const size_t row0 = (size_t(s) * p.num_q_heads + h) * p.max_parts;
  float M = kNegInf;
  for (int q = 0; q < nparts; ++q) M = fmaxf(M, p.ws_ml[(row0 + q) * 2]);
  float num = 0.f, den = 0.f;
  for (int q = 0; q < nparts; ++q) {
    const float w = p.ws_ml[(row0 + q) * 2 + 1] * exp2f(p.ws_ml[(row0 + q) * 2] - M);
    num += w * p.ws_o[(row0 + q) * D + d];
    den += w;
  }
  store_out(p, s, h, d, num / den);
}

// ---------------------------------------------------------------------------
// slot-mapped append
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int i = blockIdx.x;
  const int64_t slot = p.slots[i];
  if (slot < 0) return;
  const int64_t blk = slot / BS;
  const int off = int(slot - blk * BS);
  const int units = p.num_kv_heads * (D / 8);
  for (int u = blockIdx.y * blockDim.x + threadIdx.x; u < units; u += gridDim.y * blockDim.x) {
    const int h = u / (D / 8);
    const int piece = u - h * (D / 8);
    const u32x4 kv = load16(p.k + size_t(i) * p.k_t + size_t(h) * p.k_h + piece * 8);
    const u32x4 vv = load16(p.v + size_t(i) * p.v_t + size_t(h) * p.v_h + piece * 8);
    const size_t tile = (size_t(blk) * p.num_kv_heads + h) * (BS * D);
    store16(p.k_cache + tile + (piece * BS + off) * 8, kv);
    uint16_t* vt = p.v_cache + tile + ((off >> 2) * D + piece * 8) * 4 + (off & 3);
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(2 * e) * 4] = uint16_t(w[e] & 0xffffu);
      vt[(2 * e + 1) * 4] = uint16_t(w[e] >> 16);
    }
  }
}

template <int D, int BS>
hipError_t launch_decode_t(const DecodeParams& p, Path path, hipStream_t stream) {
  const dim3 block(kThreads);
  if (path == Path::Mfma) {
    const dim3 grid(p.num_kv_heads * p.head_groups, p.num_seqs, p.max_parts);
    hipLaunchKernelGGL((decode_mfma<D, BS>), grid, block, 0, stream, p);
  } else {
    const dim3 grid(p.num_kv_heads, p.num_seqs, p.max_parts);
    if (p.group == 1)
      hipLaunchKernelGGL((decode_valu<D, BS, 1>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_valu<D, BS, 2>), grid, block, 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_parts <= 1) return e;
  const dim3 cgrid((p.num_q_heads * D + 255) / 256, p.num_seqs);
  hipLaunchKernelGGL((combine_kernel<D>), cgrid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, int block_size, Path path, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_decode_t<D, 8>(p, path, stream);
    case 16: return launch_decode_t<D, 16>(p, path, stream);
    case 32: return launch_decode_t<D, 32>(p, path, stream);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_append_d(const AppendParams& p, int block_size, hipStream_t stream) {
  const int units = p.num_kv_heads * (D / 8);
  const dim3 grid(p.num_tokens, (units + 255) / 256);
  const dim3 block(256);
  switch (block_size) {
    case 8: hipLaunchKernelGGL((append_kernel<D, 8>), grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL((append_kernel<D, 16>), grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL((append_kernel<D, 32>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, int block_size, Path path,
                         hipStream_t stream) {
  if (head_dim == 64) return launch_decode_d<64>(p, block_size, path, stream);
  if (head_dim == 128) return launch_decode_d<128>(p, block_size, path, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_append(const AppendParams& p, int head_dim, int block_size, hipStream_t stream) {
  if (head_dim == 64) return launch_append_d<64>(p, block_size, stream);
  if (head_dim == 128) return launch_append_d<128>(p, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
