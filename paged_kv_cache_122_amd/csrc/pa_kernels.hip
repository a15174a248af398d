// HIP kernels for gfx950 (CDNA4): slot-mapped KV append and paged decode
// attention with a fused split-K log-sum-exp combine.
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
// * Work unit = (kv head [x column group], sequence, 512-token partition); a
//   workgroup of 4 wave64s, each wave walking every 4th 16-token tile of the
//   partition with the next tile's loads in flight while it computes on the
//   current one.
// * Pool layouts (K [NB, Hkv, D/8, B, 8], V [NB, Hkv, B/4, D, 4]) make every
//   16-byte lane load land directly in MFMA operand order, 256 contiguous
//   bytes per 16 lanes, so there is no LDS staging of K/V and no shuffles
//   before the matrix cores.
// * GQA path (q heads per KV head >= 3): QK^T is v_mfma_f32_16x16x32_bf16 with
//   16 tokens as rows and the group's query heads as columns; PV is
//   v_mfma_f32_16x16x16_bf16 whose B operand is exactly the QK^T accumulator
//   layout, so probabilities go from scores to PV without moving between
//   lanes.  P is split into a high and a low bf16 part (two MFMAs) so the PV
//   product keeps ~16 significant bits of P.
// * MHA path (1 or 2 q heads per KV head): fp32 FMAs on the same loads,
//   cross-lane sums with wave shuffles.
// * Split-K combine fused into the decode kernel: each partition writes
//   (max, sum, normalised output) to a workspace and bumps a per-(sequence,
//   head) counter; the workgroup that finishes last combines the partitions
//   in ascending order (deterministic) and resets the counter.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_internal.h"

namespace pa {

WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                                 int64_t head_dim, int64_t max_parts) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const int64_t group = num_q_heads / num_kv_heads;
  const int64_t head_groups = (group + 15) / 16;
  WorkspaceLayout w;
  w.count_off = 0;
  w.ml_off = up(sizeof(int32_t) * size_t(num_seqs * num_kv_heads * head_groups));
  w.o_off = w.ml_off + up(sizeof(float) * 2 * size_t(num_seqs * num_q_heads * max_parts));
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

// Per-lane base pointers of one 16-token tile.
//
// K: lane l holds token row r = l & 15 and, for chunk c, dims
//    8*((l >> 4) + 4c) .. +7 -- one 16-byte load per chunk.
// V: lane l holds tokens 4*(l >> 4) .. +3 and, for chunk c, dims
//    2*(l & 15) + 32c and the next one -- one 16-byte load per chunk.
template <int D, int BS>
struct TileAddr {
  const uint16_t* k;
  const uint16_t* v;
};

template <int D, int BS>
__device__ __forceinline__ TileAddr<D, BS> tile_addr(const DecodeParams& p, const int32_t* bt,
                                                     int kvh, int ts, int t1, int lane) {
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const size_t blk_elems = size_t(p.num_kv_heads) * BS * D;
  const size_t head_off = size_t(kvh) * BS * D;
  TileAddr<D, BS> a;
  if constexpr (BS == 16) {
    const size_t base = size_t(bt[ts >> 4]) * blk_elems + head_off;
    a.k = p.k_cache + base + (g4 * BS + r) * 8;
    a.v = p.v_cache + base + (g4 * D + 2 * r) * 4;
  } else if constexpr (BS == 32) {
    const size_t base = size_t(bt[ts >> 5]) * blk_elems + head_off;
    const int half = (ts >> 4) & 1;
    a.k = p.k_cache + base + (g4 * BS + 16 * half + r) * 8;
    a.v = p.v_cache + base + ((g4 + 4 * half) * D + 2 * r) * 4;
  } else {  // BS == 8: the tile spans two blocks; the second may lie past the context
    const int b0 = ts >> 3;
    const int phys0 = bt[b0];
    const int phys1 = (ts + 8 < t1) ? bt[b0 + 1] : phys0;
    const size_t base0 = size_t(phys0) * blk_elems + head_off;
    const size_t base1 = size_t(phys1) * blk_elems + head_off;
    a.k = p.k_cache + ((r >> 3) ? base1 : base0) + (g4 * BS + (r & 7)) * 8;
    a.v = p.v_cache + ((g4 >> 1) ? base1 : base0) + ((g4 & 1) * D + 2 * r) * 4;
  }
  return a;
}

template <int D, int BS>
__device__ __forceinline__ void load_tile(const TileAddr<D, BS>& a, u32x4 (&k)[D / 32],
                                          u32x4 (&v)[D / 32]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) k[c] = load16(a.k + c * 4 * BS * 8);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) v[c] = load16(a.v + c * 128);
}

// Zero the V values of tokens at or past t1 (0 * NaN would poison the sum).
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
  int last;
};

// Combine the waves' (m, l, o) and either write the output (one partition) or
// the partition's partial result, then -- for split contexts -- let the last
// workgroup of the (sequence, head group) combine all partitions.
template <int D>
__device__ __forceinline__ void finish(const DecodeParams& p, Smem<D>& sm, int s, int hg, int h0,
                                       int ncols, int part, int nparts) {
  __syncthreads();
  const bool split = nparts > 1;
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
    if (!split) {
      const float r = l > 0.f ? o / l : 0.f;
      if (p.out_f32)
        static_cast<float*>(p.out)[size_t(s) * p.out_s + size_t(h) * p.out_h + d] = r;
      else
        static_cast<uint16_t*>(p.out)[size_t(s) * p.out_s + size_t(h) * p.out_h + d] =
            uint16_t(bf16_bits(r));
    } else {
      const size_t row = (size_t(s) * p.num_q_heads + h) * p.max_parts + part;
      p.ws_o[row * D + d] = o / l;
      if (d == 0) {
        p.ws_ml[row * 2 + 0] = M;
        p.ws_ml[row * 2 + 1] = l;
      }
    }
  }
  if (!split) return;

  __syncthreads();
  int32_t* counter = p.ws_count + size_t(s) * gridDim.x + hg;
  if (threadIdx.x == 0) {
    __threadfence();  // release this partition's partials, device-wide
    const int prev = atomicAdd(counter, 1);
    sm.last = (prev == nparts - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  __threadfence();  // acquire every partition's partials

  for (int idx = threadIdx.x; idx < ncols * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    const size_t row0 = (size_t(s) * p.num_q_heads + h0 + g) * p.max_parts;
    float M = kNegInf;
    for (int q = 0; q < nparts; ++q) M = fmaxf(M, p.ws_ml[(row0 + q) * 2]);
    float num = 0.f, den = 0.f;
    for (int q = 0; q < nparts; ++q) {
      const float w = p.ws_ml[(row0 + q) * 2 + 1] * exp2f(p.ws_ml[(row0 + q) * 2] - M);
      num += w * p.ws_o[(row0 + q) * D + d];
      den += w;
    }
    const float r = num / den;
    const int h = h0 + g;
    if (p.out_f32)
      static_cast<float*>(p.out)[size_t(s) * p.out_s + size_t(h) * p.out_h + d] = r;
    else
      static_cast<uint16_t*>(p.out)[size_t(s) * p.out_s + size_t(h) * p.out_h + d] =
          uint16_t(bf16_bits(r));
  }
  if (threadIdx.x == 0) atomicExch(counter, 0);
}

// ---------------------------------------------------------------------------
// GQA decode on the matrix cores
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_mfma(DecodeParams p) {
  constexpr int NC = D / 32;  // 16-byte chunks per lane per tile, for K and for V
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int hg = blockIdx.x;
  const int kvh = hg / p.head_groups;
  const int cgrp = hg - kvh * p.head_groups;
  const int s = blockIdx.y;
  const int part = blockIdx.z;

  const int L = p.context_lens[s];
  // contexts longer than the launch covers violate the caller's contract; clamp
  // so that the partition count stays consistent with the grid
  const int nparts = min((L + p.part_tokens - 1) / p.part_tokens, p.max_parts);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int t0 = part * p.part_tokens;
  const int t1 = min(L, t0 + p.part_tokens);
  const int ntiles = (t1 - t0 + 15) >> 4;
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
  float m_run = kNegInf;  // running max (log2 units) of column r
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
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float pr[4];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[j] = exp2f(sc[j] - m_new);
      psum += pr[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) oacc[i] *= alpha;
    // P as the B operand of PV, split into hi + lo bf16
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hb[j] = bf16_bits(pr[j]);
      lb[j] = bf16_bits(pr[j] - bf16_value(hb[j]));
    }
    const u32x2 phi = {hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    const u32x2 plo = {lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
    if (ts + 16 > t1) mask_v<D>(vt, ts, t1, lane);
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

  u32x4 ka[NC], va[NC], kb[NC], vb[NC];
  int i = wave;
  if (i < ntiles) load_tile<D, BS>(tile_addr<D, BS>(p, bt, kvh, t0 + 16 * i, t1, lane), ka, va);
  while (i < ntiles) {
    int in = i + kWaves;
    if (in < ntiles) load_tile<D, BS>(tile_addr<D, BS>(p, bt, kvh, t0 + 16 * in, t1, lane), kb, vb);
    compute(t0 + 16 * i, ka, va);
    i = in;
    if (i >= ntiles) break;
    in = i + kWaves;
    if (in < ntiles) load_tile<D, BS>(tile_addr<D, BS>(p, bt, kvh, t0 + 16 * in, t1, lane), ka, va);
    compute(t0 + 16 * i, kb, vb);
    i = in;
  }

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

  finish<D>(p, sm, s, hg, h0, ncols, part, nparts);
}

// ---------------------------------------------------------------------------
// MHA decode (1 or 2 query heads per KV head) on the vector ALUs
// ---------------------------------------------------------------------------
template <int D, int BS, int VG>
__global__ __launch_bounds__(kThreads) void decode_valu(DecodeParams p) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int part = blockIdx.z;

  const int L = p.context_lens[s];
  // contexts longer than the launch covers violate the caller's contract; clamp
  // so that the partition count stays consistent with the grid
  const int nparts = min((L + p.part_tokens - 1) / p.part_tokens, p.max_parts);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int t0 = part * p.part_tokens;
  const int t1 = min(L, t0 + p.part_tokens);
  const int ntiles = (t1 - t0 + 15) >> 4;
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
    if (ts + 16 > t1) mask_v<D>(vt, ts, t1, lane);
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
      const float m_new = fmaxf(m_run[g], mt);
      const float alpha = exp2f(m_run[g] - m_new);
      const float pr = exp2f(sc - m_new);
      l_run[g] = l_run[g] * alpha + pr;
      m_run[g] = m_new;
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

  u32x4 ka[NC], va[NC], kb[NC], vb[NC];
  int i = wave;
  if (i < ntiles) load_tile<D, BS>(tile_addr<D, BS>(p, bt, kvh, t0 + 16 * i, t1, lane), ka, va);
  while (i < ntiles) {
    int in = i + kWaves;
    if (in < ntiles) load_tile<D, BS>(tile_addr<D, BS>(p, bt, kvh, t0 + 16 * in, t1, lane), kb, vb);
    compute(t0 + 16 * i, ka, va);
    i = in;
    if (i >= ntiles) break;
    in = i + kWaves;
    if (in < ntiles) load_tile<D, BS>(tile_addr<D, BS>(p, bt, kvh, t0 + 16 * in, t1, lane), ka, va);
    compute(t0 + 16 * i, kb, vb);
    i = in;
  }

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

  finish<D>(p, sm, s, kvh, h0, VG, part, nparts);
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

__global__ __launch_bounds__(256) void zero_kernel(int32_t* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0;
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

hipError_t launch_zero(int32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = unsigned(std::min<size_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace pa
