// HIP kernels for gfx950 (CDNA4): slot-mapped KV append, paged decode
// attention, the split-K log-sum-exp combine, batched copy-on-write block
// copies, and attention for several new tokens per sequence with their
// append fused in (chunked prefill, speculative verification, and the
// one-launch decode step).
//
// Method: one query token per sequence attends to its cached tokens, which
// live in fixed-size physical blocks reached through a per-sequence block
// table; the per-block softmax is accumulated online (running max and sum,
// rescaled when the max grows) and, for long contexts, partial results of
// pieces of the context are combined by a reduce step ("PagedAttention from
// First Principles", sections 5 and 17; Equation 4 of the hungchun0201 vLLM
// digest).  The pages' kernel sketch (one warp per block, reduce across warps)
// targets other hardware; the design here is gfx950's:
//
// * Unit of work: one 16-token tile of one (sequence, KV head [x column
//   group]) pair.  Lane layouts make every 16-byte lane load land directly in
//   MFMA operand order (pool layouts K [NB, Hkv, D/8, B, 8], V [NB, Hkv, B/4,
//   D, 4]; 256 contiguous bytes per 16 lanes), so K/V go from HBM to the
//   matrix cores without LDS staging or shuffles.
// * Loads are buffer loads through a resource descriptor built per tile in
//   scalar registers from the block-table entry, with the non-temporal bit
//   (the pools are read once per step).  Each wave keeps the next tile's loads
//   in flight while it computes on the current one (the next three on grids
//   of fewer workgroups than compute units, which are latency-bound); past its
//   last tile a zero-record descriptor turns the padding loads into free zero
//   loads, so the loop never branches around a load and the compiler waits
//   only for the tile it is about to use.
// * Partitioned schedule: a grid of (pair, partition) workgroups of 4 waves,
//   each wave walking every 4th tile of its partition.  Unsplit grids hand
//   their rows to the sequences by rank of context length (longest first, or
//   long paired with short on each compute unit when the whole grid is
//   resident), so no compute unit is left with the longest work at the end.
//   Split grids read a partition that neighbouring sequences fill with the
//   same blocks (a shared prefix) once, for all of them.
// * Stream-K schedule (few long contexts): the tiles of all pairs, in
//   (sequence, head, tile) order, are cut into one equal contiguous range per
//   wave of a persistent grid (a few workgroups per CU), so every wave streams
//   the same number of bytes whatever the length mix, pays its start-up
//   latency once, and keeps its pipeline full across pair boundaries.  A pair
//   finished inside one wave is written out directly; a pair cut between waves
//   leaves one partial result per wave for the combine kernel.
// * GQA path (q heads per KV head >= 3): QK^T is v_mfma_f32_16x16x32_bf16 with
//   16 tokens as rows and the group's query heads as columns.  PV is the same
//   instruction with V rows as A and P as B: a lane's P values sit exactly where
//   the QK^T accumulator left them, so probabilities go from scores to PV
//   without moving between lanes.  P is split into a high and a low bf16 part,
//   placed in the two halves of each lane's eight k values against the same
//   four V values twice, so the PV product keeps ~16 significant bits of P at
//   one MFMA per accumulator.
// * MHA path (1 or 2 q heads per KV head, unsplit): fp32 FMAs on the same
//   loads, cross-lane sums with wave shuffles.
// * Several new tokens per sequence: MFMA columns are (new token, query head)
//   pairs, causal among the new tokens, whose K/V are read from the inputs
//   and stored to their slots after the cached context has been read.
// * The softmax reference max is raised lazily: only when a tile's max
//   exceeds it by more than 2^8 in probability, so the accumulator rescale
//   runs on a handful of tiles instead of every tile.  Numerator and
//   denominator share the reference, so the result is the same quantity.
// * Combine: out = sum_p w_p o_p / sum_p w_p with w_p = l_p 2^(m_p - M) over
//   the pieces of a pair in ascending token order (deterministic).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_map>

#include "pa.h"
#include "pa_internal.h"

// Partial results of pa_decode_noalloc's split schedules: each GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// stands for no device address; the launchers use the address that
// noalloc_scratch() looks up per device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;  // device -> its copy of the array
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  *bytes = PA_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                                 int64_t max_parts) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WorkspaceLayout w;
  w.plan_off = 0;
  w.ml_off = 0;
  w.o_off = up(sizeof(float) * 2 * size_t(num_seqs * num_q_heads * max_parts));
  w.total = w.o_off + up(sizeof(float) * size_t(num_seqs * num_q_heads * max_parts * head_dim));
  return w;
}

WorkspaceLayout stream_workspace_layout(int64_t num_seqs, int64_t num_pairs, int64_t head_dim) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t pieces = size_t(num_pairs + kMaxStreamWaves);
  WorkspaceLayout w;
  w.plan_off = 0;
  w.ml_off = up(sizeof(int32_t) * size_t(num_seqs + 1 + kPlanHeader));
  w.o_off = w.ml_off + up(sizeof(float) * 2 * pieces * 16);
  w.total = w.o_off + up(sizeof(float) * pieces * 16 * size_t(head_dim));
  return w;
}

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();
// gfx9 buffer descriptor word 3 for raw dword access
constexpr int kBufferFlags = 0x00020000;
// a byte offset no tile reaches: buffer loads at it return zeros, touching no memory
constexpr uint32_t kOutOfRange = 0x80000000u;
// lazy rescale threshold (log2 units): probabilities stay <= 2^8
constexpr float kRescaleSlack = 8.f;
// K/V tiles are read once per decode step: non-temporal loads (the nt bit)
// stream them without displacing cached data, and on MI355X sustain ~25 %
// more HBM read bandwidth than default-policy loads for 4 KiB random tiles.
constexpr int kStreamingLoad = 2;

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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}
// o0 (dim 2r + 32c) and o1 (dim 2r + 32c + 1) += V P for one tile, as four
// K = 16 MFMAs: this lane's V of tokens 4*g4 .. +3 straight from the loaded
// registers (x, y: dim 2r + 32c; z, w: the next dim), P's hi then lo halves.
// One K = 32 MFMA per dim would need V repeated in an operand quad; the
// copies that builds keep the register allocator from holding the next
// tile's loads in flight across the softmax (it waits for every load).
__device__ __forceinline__ void pv16(f32x4& o0, f32x4& o1, u32x4 v, u32x4 pb) {
  const u32x2 vx = {v.x, v.y}, vz = {v.z, v.w}, ph = {pb.x, pb.y}, pl = {pb.z, pb.w};
  o0 = mfma_16x16x16(vx, ph, o0);
  o1 = mfma_16x16x16(vz, ph, o1);
  o0 = mfma_16x16x16(vx, pl, o0);
  o1 = mfma_16x16x16(vz, pl, o1);
}

__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

// 2^x with the hardware instruction: results below 2^-126 flush to zero,
// which a softmax probability can lose (it is then below the fp32 resolution
// of the running sum), and 2^-inf = 0.
__device__ __forceinline__ float exp2_ftz(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ u32x4 stream_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kStreamingLoad));
}

__device__ __forceinline__ u32x4 cached_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}

__device__ __forceinline__ void store_out(const DecodeParams& p, int s, int h, int d, float r) {
  const size_t at = size_t(s) * p.out_s + size_t(h) * p.out_h + d;
  if (p.out_f32)
    static_cast<float*>(p.out)[at] = r;
  else
    static_cast<uint16_t*>(p.out)[at] = uint16_t(bf16_bits(r));
}

// Dims d0 .. d0 + 7 of output row (s, h) in one 16-byte store (two for f32
// outputs) where the row starts 16-byte aligned, element by element otherwise
// (strided outputs).  d0 is a multiple of 8.
__device__ __forceinline__ void store_out8(const DecodeParams& p, int s, int h, int d0, const float (&o)[8]) {
  const size_t at = size_t(s) * p.out_s + size_t(h) * p.out_h + d0;
  if (p.out_f32) {
    float* dst = static_cast<float*>(p.out) + at;
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = o[j];
    }
  } else {
    uint16_t* dst = static_cast<uint16_t*>(p.out) + at;
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
      store16(dst, u32x4{bf16_bits(o[0]) | (bf16_bits(o[1]) << 16), bf16_bits(o[2]) | (bf16_bits(o[3]) << 16),
                         bf16_bits(o[4]) | (bf16_bits(o[5]) << 16), bf16_bits(o[6]) | (bf16_bits(o[7]) << 16)});
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = uint16_t(bf16_bits(o[j]));
    }
  }
}

// Context length as the kernels use it: negative lengths count as 0 and
// lengths past the block table (a contract violation) are clamped to it.
__device__ __forceinline__ int clamp_len(const DecodeParams& p, int L) {
  return min(max(L, 0), p.max_len);
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

// Load the tile starting at token ts of KV head kvh whose physical block(s)
// are phys0 / phys1, or zeros without any memory access when !valid.  Lanes
// whose tokens (K row, or first token of the V quad) lie at or past t1 load
// zeros through an out-of-range offset, so the last tile of a context reads
// only its live rows.
template <int D, int BS>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int kvh, int phys0, int phys1,
                                          int ts, int t1, bool valid, const LaneOffsets<D, BS>& lo,
                                          u32x4 (&k)[D / 32], u32x4 (&v)[D / 32]) {
  constexpr int kTileBytes = BS * D * 2;
  const int lane = __lane_id();
  const uint32_t kx = ts + (lane & 15) >= t1 ? kOutOfRange : 0u;
  const uint32_t vx = ts + 4 * (lane >> 4) >= t1 ? kOutOfRange : 0u;
  const size_t blk_elems = size_t(p.num_kv_heads) * BS * D;
  const size_t head_off = size_t(kvh) * BS * D;
  const int bytes = valid ? kTileBytes : 0;
  const auto k0 = make_rsrc(p.k_cache + size_t(phys0) * blk_elems + head_off, bytes);
  const auto v0 = make_rsrc(p.v_cache + size_t(phys0) * blk_elems + head_off, bytes);
  if constexpr (BS == 8) {
    const auto k1 = make_rsrc(p.k_cache + size_t(phys1) * blk_elems + head_off, bytes);
    const auto v1 = make_rsrc(p.v_cache + size_t(phys1) * blk_elems + head_off, bytes);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      k[c] = stream_load16(k0, (lo.k0 + c * 4 * BS * 16) | kx) | stream_load16(k1, (lo.k1 + c * 4 * BS * 16) | kx);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      v[c] = stream_load16(v0, (lo.v0 + c * 256) | vx) | stream_load16(v1, (lo.v1 + c * 256) | vx);
  } else {
    // B = 32 holds two tiles per block: the second half starts 16 tokens in
    const uint32_t khalf = BS == 32 ? uint32_t(((ts >> 4) & 1) * 16 * 8 * 2) : 0u;
    const uint32_t vhalf = BS == 32 ? uint32_t(((ts >> 4) & 1) * 4 * D * 4 * 2) : 0u;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) k[c] = stream_load16(k0, (lo.k0 + khalf + c * 4 * BS * 16) | kx);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) v[c] = stream_load16(v0, (lo.v0 + vhalf + c * 256) | vx);
  }
}

// Physical block(s) of tile t (tokens 16t .. 16t+15) of a sequence with L
// tokens; for B = 8 the second block is the first again when it lies past L.
template <int BS>
__device__ __forceinline__ void tile_blocks(const int32_t* bt_row, int t, int L, int& b0, int& b1) {
  if constexpr (BS == 16) {
    b0 = bt_row[t];
    b1 = 0;
  } else if constexpr (BS == 32) {
    b0 = bt_row[t >> 1];
    b1 = 0;
  } else {
    b0 = bt_row[2 * t];
    b1 = (16 * t + 8 < L) ? bt_row[2 * t + 1] : b0;
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

// ---------------------------------------------------------------------------
// per-tile math, GQA path (MFMA)
//
// Column r of the accumulators is query head h0 + r.  Lane (g4 = l >> 4, r)
// holds the scores of tokens 4*g4 .. +3 of the tile and the output rows
// d = 2*(4*g4 + j) + 32*(mm >> 1) + (mm & 1) of accumulator mm.
// ---------------------------------------------------------------------------
template <int D>
struct MfmaAcc {
  f32x4 o[D / 16];
  float m;  // reference max (log2 units) of column r
  float l;  // this lane's share of the running sum of column r
};

template <int D>
__device__ __forceinline__ void mfma_reset(MfmaAcc<D>& a) {
#pragma unroll
  for (int i = 0; i < D / 16; ++i) a.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  a.m = kNegInf;
  a.l = 0.f;
}

// Scores of one tile (QK^T), the online-softmax update of the column
// references and sums, and P as the B operand of PV, split into hi + lo
// bf16: x, y the high halves of this lane's four tokens, z, w the low ones
// (pv16 takes each pair against the same V registers).
template <int D>
__device__ __forceinline__ u32x4 mfma_probs(MfmaAcc<D>& a, const u32x4 (&q)[D / 32], float scale_log2,
                                            bool partial, int ts, int t1, int lane,
                                            const u32x4 (&kt)[D / 32]) {
  constexpr int NC = D / 32;
  const int g4 = lane >> 4;
  // two independent accumulation chains, so the QK^T MFMAs overlap
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; c += 2) {
    s0 = mfma_16x16x32(kt[c], q[c], s0);
    s1 = mfma_16x16x32(kt[c + 1], q[c + 1], s1);
  }
  const f32x4 sacc = s0 + s1;
  float sc[4];
  float mt = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sc[j] = sacc[j] * scale_log2;
    if (partial && ts + 4 * g4 + j >= t1) sc[j] = kNegInf;
    mt = fmaxf(mt, sc[j]);
  }
  // Raise the reference only when some score is far above it; the column max
  // (over the four 16-lane groups) is needed only then.
  if (__any(mt > a.m + kRescaleSlack)) {
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(a.m, mt);
    const float alpha = exp2_ftz(a.m - m_new);
    a.l *= alpha;
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) a.o[i] *= alpha;
    a.m = m_new;
  }
  float pr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr[j] = exp2_ftz(sc[j] - a.m);
    a.l += pr[j];
  }
  uint32_t hb[4], lb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hb[j] = bf16_bits(pr[j]);
    lb[j] = bf16_bits(pr[j] - bf16_value(hb[j]));
  }
  return u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
}

template <int D>
__device__ __forceinline__ void mfma_tile(MfmaAcc<D>& a, const u32x4 (&q)[D / 32], float scale_log2,
                                          int ts, int t1, int lane, u32x4 (&kt)[D / 32],
                                          u32x4 (&vt)[D / 32]) {
  constexpr int NC = D / 32;
  // Only the last tile of a context has tokens at or past t1 (wave-uniform
  // test): the others skip the score and V masks.
  const bool partial = ts + kTileTokens > t1;
  const u32x4 pb = mfma_probs<D>(a, q, scale_log2, partial, ts, t1, lane, kt);
  if (partial) mask_v<D>(vt, ts, t1, lane);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    pv16(a.o[2 * c], a.o[2 * c + 1], vt[c], pb);
  }
}

// mfma_tile for NS sets of 16 columns against one tile: each V operand is
// built once and feeds every set.
template <int D, int NS>
__device__ __forceinline__ void mfma_tile_sets(MfmaAcc<D> (&a)[NS], const u32x4 (&q)[NS][D / 32],
                                               float scale_log2, int ts, int t1, int lane,
                                               u32x4 (&kt)[D / 32], u32x4 (&vt)[D / 32]) {
  constexpr int NC = D / 32;
  const bool partial = ts + kTileTokens > t1;
  u32x4 pb[NS];
#pragma unroll
  for (int cs = 0; cs < NS; ++cs) pb[cs] = mfma_probs<D>(a[cs], q[cs], scale_log2, partial, ts, t1, lane, kt);
  if (partial) mask_v<D>(vt, ts, t1, lane);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int cs = 0; cs < NS; ++cs) pv16(a[cs].o[2 * c], a[cs].o[2 * c + 1], vt[c], pb[cs]);
  }
}

// mfma_probs with a per-column limit: token tok0 + 4*g4 + j counts for this
// lane's column when it is at most climit (new tokens: the column's query
// index; a run's tile: the tile's end for the columns it counts for, -1 for
// the others).  Masked scores contribute exactly zero even before the column
// has seen a token.
template <int D>
__device__ __forceinline__ u32x4 mfma_probs_limit(MfmaAcc<D>& a, const u32x4 (&q)[D / 32], float scale_log2,
                                                  int tok0, int climit, int lane, const u32x4 (&kt)[D / 32]) {
  constexpr int NC = D / 32;
  const int g4 = lane >> 4;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; c += 2) {
    s0 = mfma_16x16x32(kt[c], q[c], s0);
    s1 = mfma_16x16x32(kt[c + 1], q[c + 1], s1);
  }
  const f32x4 sacc = s0 + s1;
  float sc[4];
  bool vis[4];
  float mt = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vis[j] = tok0 + 4 * g4 + j <= climit;
    sc[j] = vis[j] ? sacc[j] * scale_log2 : kNegInf;
    mt = fmaxf(mt, sc[j]);
  }
  if (__any(mt > a.m + kRescaleSlack)) {
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(a.m, mt);
    const float alpha = a.m == kNegInf ? 0.f : exp2_ftz(a.m - m_new);
    a.l *= alpha;
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) a.o[i] *= alpha;
    a.m = m_new;
  }
  float pr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr[j] = vis[j] ? exp2_ftz(sc[j] - a.m) : 0.f;
    a.l += pr[j];
  }
  uint32_t hb[4], lb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hb[j] = bf16_bits(pr[j]);
    lb[j] = bf16_bits(pr[j] - bf16_value(hb[j]));
  }
  return u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
}

// o += P V for one tile, P as mfma_probs returns it (hi + lo bf16).
template <int D>
__device__ __forceinline__ void mfma_pv(MfmaAcc<D>& a, u32x4 pb, const u32x4 (&vt)[D / 32]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    pv16(a.o[2 * c], a.o[2 * c + 1], vt[c], pb);
  }
}

// mfma_tile with a per-column limit (mfma_probs_limit).  V past the tile's
// tokens must be finite (zeros).
template <int D>
__device__ __forceinline__ void mfma_tile_causal(MfmaAcc<D>& a, const u32x4 (&q)[D / 32], float scale_log2,
                                                 int tok0, int climit, int lane, const u32x4 (&kt)[D / 32],
                                                 const u32x4 (&vt)[D / 32]) {
  mfma_pv<D>(a, mfma_probs_limit<D>(a, q, scale_log2, tok0, climit, lane, kt), vt);
}

// ---------------------------------------------------------------------------
// per-tile math, MHA path (VALU)
//
// Lane (g4, r) holds token r of the tile and dims 8*(g4 + 4c) .. +7 of K, and
// output dims 2r + 32c + e (summed over the four 16-lane groups at the end).
// ---------------------------------------------------------------------------
template <int D, int VG>
struct ValuAcc {
  float o[VG][D / 32][2];
  float m[VG];  // reference max, the same in every lane
  float l[VG];  // this lane's share: the probabilities of its token
};

template <int D, int VG>
__device__ __forceinline__ void valu_reset(ValuAcc<D, VG>& a) {
#pragma unroll
  for (int g = 0; g < VG; ++g) {
    a.m[g] = kNegInf;
    a.l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) a.o[g][c][0] = a.o[g][c][1] = 0.f;
  }
}

// q in fp32: this lane's dims 8*(g4 + 4c) + e of query heads h0 .. h0+VG-1
template <int D, int VG>
__device__ __forceinline__ void valu_load_q(const DecodeParams& p, int s, int h0, int lane,
                                            float (&qf)[VG][D / 32][8]) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < VG; ++g)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const u32x4 u = load16(p.q + size_t(s) * p.q_s + size_t(h0 + g) * p.q_h + 8 * (g4 + 4 * c));
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[g][c][2 * e] = bf_lo(w[e]);
        qf[g][c][2 * e + 1] = bf_hi(w[e]);
      }
    }
}

template <int D, int VG>
__device__ __forceinline__ void valu_tile(ValuAcc<D, VG>& a, const float (&qf)[VG][D / 32][8],
                                          float scale_log2, int ts, int t1, int lane,
                                          u32x4 (&kt)[D / 32], u32x4 (&vt)[D / 32]) {
  constexpr int NC = D / 32;
  const int r = lane & 15;
  const int g4 = lane >> 4;
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
    const float sc = valid ? dot * scale_log2 : kNegInf;  // score of token ts + r
    float mt = sc;
    mt = fmaxf(mt, shfl_xor(mt, 1));
    mt = fmaxf(mt, shfl_xor(mt, 2));
    mt = fmaxf(mt, shfl_xor(mt, 4));
    mt = fmaxf(mt, shfl_xor(mt, 8));
    float alpha = 1.f;
    if (mt > a.m[g] + kRescaleSlack) {  // the same in every lane
      const float m_new = fmaxf(a.m[g], mt);
      alpha = exp2_ftz(a.m[g] - m_new);
      a.l[g] *= alpha;
      a.m[g] = m_new;
    }
    const float pr = exp2_ftz(sc - a.m[g]);
    a.l[g] += pr;
    float pj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pj[j] = __shfl(pr, 4 * g4 + j, 64);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float a0 = a.o[g][c][0] * alpha, a1 = a.o[g][c][1] * alpha;
      a0 = fmaf(pj[0], bf_lo(vt[c].x), a0);
      a0 = fmaf(pj[1], bf_hi(vt[c].x), a0);
      a0 = fmaf(pj[2], bf_lo(vt[c].y), a0);
      a0 = fmaf(pj[3], bf_hi(vt[c].y), a0);
      a1 = fmaf(pj[0], bf_lo(vt[c].z), a1);
      a1 = fmaf(pj[1], bf_hi(vt[c].z), a1);
      a1 = fmaf(pj[2], bf_lo(vt[c].w), a1);
      a1 = fmaf(pj[3], bf_hi(vt[c].w), a1);
      a.o[g][c][0] = a0;
      a.o[g][c][1] = a1;
    }
  }
}

// ===========================================================================
// stream-K schedule
// ===========================================================================

// Exclusive prefix of tiles per sequence into LDS: ps[s] = sum_{s' < s}
// ceil(L_s' / 16), ps[S] = total.  All threads of the workgroup take part.
__device__ __forceinline__ void build_prefix(const DecodeParams& p, int* ps, int* scan) {
  const int S = p.num_seqs;
  const int per = (S + kThreads - 1) / kThreads;
  const int b = threadIdx.x * per;
  const int e = min(S, b + per);
  int sum = 0;
  for (int i = b; i < e; ++i) {
    const int n = (clamp_len(p, p.context_lens[i]) + 15) >> 4;
    ps[i] = n;
    sum += n;
  }
  scan[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {  // inclusive Hillis-Steele scan
    const int add = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  int run = threadIdx.x ? scan[threadIdx.x - 1] : 0;
  for (int i = b; i < e; ++i) {
    const int n = ps[i];
    ps[i] = run;
    run += n;
  }
  if (threadIdx.x == kThreads - 1) ps[S] = scan[kThreads - 1];
  __syncthreads();
}

// Position of global tile T: sequence s (largest with H*ps[s] <= T), head
// group hg and tile t within the pair.
__device__ __forceinline__ void locate(const int* ps, int S, int H, int T, int& s, int& hg, int& t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (H * ps[mid] <= T) lo = mid; else hi = mid - 1;
  }
  s = lo;
  const int off = T - H * ps[lo];
  const int n = ps[lo + 1] - ps[lo];
  hg = off / n;
  t = off - hg * n;
}

// Where a pair's pieces live: pieces are numbered pair + wave (unique because
// waves take increasing tile ranges), 16 columns each.
__device__ __forceinline__ size_t piece_row(int pair, int wave, int col) {
  return (size_t(pair) + size_t(wave)) * 16 + col;
}

struct StreamRange {
  int T0, T1;  // this wave's tiles [T0, T1)
  int w;       // global wave index
};

// Per-lane cache of the metadata of up to 64 consecutive tiles of the wave:
// lane j describes tile base + j.
struct TileMeta {
  int s, hg, t, L, b0, b1;
};

template <int BS>
__device__ __forceinline__ TileMeta fetch_meta(const DecodeParams& p, const int* ps, int H, int T,
                                               bool live) {
  TileMeta m{0, 0, 0, 0, 0, 0};
  if (live) {
    locate(ps, p.num_seqs, H, T, m.s, m.hg, m.t);
    m.L = clamp_len(p, p.context_lens[m.s]);
    tile_blocks<BS>(p.block_tables + size_t(m.s) * p.bt_s, m.t, m.L, m.b0, m.b1);
  }
  return m;
}

struct Uniform {
  int s, hg, t, L, b0, b1;
};

__device__ __forceinline__ Uniform read_meta(const TileMeta& m, int j) {
  return Uniform{__builtin_amdgcn_readlane(m.s, j), __builtin_amdgcn_readlane(m.hg, j),
                 __builtin_amdgcn_readlane(m.t, j), __builtin_amdgcn_readlane(m.L, j),
                 __builtin_amdgcn_readlane(m.b0, j), __builtin_amdgcn_readlane(m.b1, j)};
}

// Query heads of head group hg: h0 .. h0 + ncols - 1
__device__ __forceinline__ void head_span(const DecodeParams& p, int hg, int& kvh, int& h0, int& ncols) {
  kvh = hg / p.head_groups;
  const int cgrp = hg - kvh * p.head_groups;
  h0 = kvh * p.group + cgrp * 16;
  ncols = min(16, p.group - cgrp * 16);
}

// Q of one pair as the B operand of QK^T (column r = head h0 + r, zero past
// the group), or zeros without memory access when !valid.
template <int D>
__device__ __forceinline__ void load_q_operand(const DecodeParams& p, int s, int hg, bool valid,
                                               int lane, u32x4 (&q)[D / 32]) {
  int kvh, h0, ncols;
  head_span(p, hg, kvh, h0, ncols);
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int bytes = valid ? int(((ncols - 1) * p.q_h + D) * 2) : 0;
  const auto rs = make_rsrc(p.q + size_t(s) * p.q_s + size_t(h0) * p.q_h, bytes);
  const uint32_t off = r < ncols ? uint32_t((r * p.q_h + 8 * g4) * 2) : kOutOfRange;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) q[c] = cached_load16(rs, off + c * 64);
}

// Write one finished piece of the MFMA path: the output itself when the wave
// saw the whole pair, else a partial result (reference max, sum, o / sum).
template <int D>
__device__ __forceinline__ void mfma_write_piece(const DecodeParams& p, const StreamParams& sk,
                                                 MfmaAcc<D>& a, int s, int hg, bool whole, int w,
                                                 int lane) {
  const int r = lane & 15;
  const int g4 = lane >> 4;
  int kvh, h0, ncols;
  head_span(p, hg, kvh, h0, ncols);
  float l = a.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (r >= ncols) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (whole) {
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_out(p, s, h0 + r, 2 * (4 * g4 + j) + 32 * (mm >> 1) + (mm & 1), a.o[mm][j] * inv);
  } else {
    const int pair = s * (p.num_kv_heads * p.head_groups) + hg;
    const size_t row = piece_row(pair, w, r);
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sk.ws_o[row * D + 2 * (4 * g4 + j) + 32 * (mm >> 1) + (mm & 1)] = a.o[mm][j] * inv;
    if (g4 == 0) {
      sk.ws_ml[row * 2 + 0] = a.m;
      sk.ws_ml[row * 2 + 1] = l;
    }
  }
}

template <int D, int VG>
__device__ __forceinline__ void valu_write_piece(const DecodeParams& p, const StreamParams& sk,
                                                 ValuAcc<D, VG>& a, int s, int kvh, bool whole,
                                                 int w, int lane) {
  const int r = lane & 15;
  const int g4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < VG; ++g) {
    float l = a.l[g];
    l += shfl_xor(l, 1);
    l += shfl_xor(l, 2);
    l += shfl_xor(l, 4);
    l += shfl_xor(l, 8);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t row = piece_row(s * p.num_kv_heads + kvh, w, g);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float x = a.o[g][c][e];
        x += shfl_xor(x, 16);
        x += shfl_xor(x, 32);
        const int d = 2 * r + 32 * c + e;
        if (g4 == 0) {
          if (whole)
            store_out(p, s, kvh * VG + g, d, x * inv);
          else
            sk.ws_o[row * D + d] = x * inv;
        }
      }
    if (!whole && lane == 0) {
      sk.ws_ml[row * 2 + 0] = a.m[g];
      sk.ws_ml[row * 2 + 1] = l;
    }
  }
}

// Shared prologue of the stream-K kernels: tile prefix in LDS, this wave's
// range, and (workgroup 0) the plan the combine kernel reads.
__device__ __forceinline__ StreamRange stream_prologue(const DecodeParams& p, const StreamParams& sk,
                                                       int* ps, int* scan, int wave) {
  build_prefix(p, ps, scan);
  const int S = p.num_seqs;
  const int H = p.num_kv_heads * p.head_groups;
  const int total = H * ps[S];
  const int nw = gridDim.x * kWaves;
  const int per = (total + nw - 1) / nw;
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= S; i += kThreads) sk.plan[kPlanHeader + i] = ps[i];
    if (threadIdx.x == 0) {
      sk.plan[0] = per;
      sk.plan[1] = total;
    }
  }
  StreamRange rg;
  rg.w = blockIdx.x * kWaves + wave;
  rg.T0 = min(rg.w * per, total);
  rg.T1 = min(rg.T0 + per, total);
  return rg;
}

template <int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_mfma_sk(DecodeParams p, StreamParams sk) {
  constexpr int NC = D / 32;
  __shared__ int ps[kMaxStreamSeqs + 1];
  __shared__ int scan[kThreads];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const StreamRange rg = stream_prologue(p, sk, ps, scan, wave);
  if (rg.T0 >= rg.T1) return;
  const int H = p.num_kv_heads * p.head_groups;
  const LaneOffsets<D, BS> lo = lane_offsets<D, BS>(lane);

  MfmaAcc<D> acc;
  mfma_reset(acc);
  u32x4 qcur[NC];
  int cur_s = -1, cur_hg = 0, cur_t0 = 0, cur_tlast = 0, cur_L = 0;

  auto finish = [&]() {
    const bool whole = cur_t0 == 0 && cur_tlast == ((cur_L + 15) >> 4) - 1;
    mfma_write_piece<D>(p, sk, acc, cur_s, cur_hg, whole, rg.w, lane);
  };

  for (int base = rg.T0; base < rg.T1; base += 64) {
    const int m = min(64, rg.T1 - base);
    const TileMeta meta = fetch_meta<BS>(p, ps, H, base + lane, lane < m);
    // load tile j of the chunk into a pipeline slot, with the pair's Q when
    // the tile opens a pair (zero-record loads otherwise and past the end)
    auto load = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC], u32x4(&qt)[NC]) {
      const int jj = min(j, m - 1);
      const Uniform u = read_meta(meta, jj);
      int kvh, h0, ncols;
      head_span(p, u.hg, kvh, h0, ncols);
      const bool opens = j < m && (u.t == 0 || base + jj == rg.T0);
      load_tile<D, BS>(p, kvh, u.b0, u.b1, 16 * u.t, u.L, j < m, lo, kt, vt);
      load_q_operand<D>(p, u.s, u.hg, opens, lane, qt);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC], u32x4(&qt)[NC]) {
      const Uniform u = read_meta(meta, j);
      if (u.t == 0 || base + j == rg.T0) {  // the tile opens a pair (or this wave's range)
        if (cur_s >= 0) finish();
        mfma_reset(acc);
#pragma unroll
        for (int c = 0; c < NC; ++c) qcur[c] = qt[c];
        cur_s = u.s;
        cur_hg = u.hg;
        cur_t0 = u.t;
        cur_L = u.L;
      }
      cur_tlast = u.t;
      mfma_tile<D>(acc, qcur, p.scale_log2, 16 * u.t, u.L, lane, kt, vt);
    };
    u32x4 ak[NC], av[NC], aq[NC], bk[NC], bv[NC], bq[NC], ck[NC], cv[NC], cq[NC];
    load(0, ak, av, aq);
    load(1, bk, bv, bq);
    for (int j = 0;; j += 3) {
      load(j + 2, ck, cv, cq);
      compute(j, ak, av, aq);
      if (j + 1 >= m) break;
      load(j + 3, ak, av, aq);
      compute(j + 1, bk, bv, bq);
      if (j + 2 >= m) break;
      load(j + 4, bk, bv, bq);
      compute(j + 2, ck, cv, cq);
      if (j + 3 >= m) break;
    }
  }
  finish();
}

template <int D, int BS, int VG>
__global__ __launch_bounds__(kThreads) void decode_valu_sk(DecodeParams p, StreamParams sk) {
  constexpr int NC = D / 32;
  __shared__ int ps[kMaxStreamSeqs + 1];
  __shared__ int scan[kThreads];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const StreamRange rg = stream_prologue(p, sk, ps, scan, wave);
  if (rg.T0 >= rg.T1) return;
  const int H = p.num_kv_heads;
  const LaneOffsets<D, BS> lo = lane_offsets<D, BS>(lane);

  ValuAcc<D, VG> acc;
  valu_reset(acc);
  float qf[VG][NC][8];
  int cur_s = -1, cur_kvh = 0, cur_t0 = 0, cur_tlast = 0, cur_L = 0;

  auto finish = [&]() {
    const bool whole = cur_t0 == 0 && cur_tlast == ((cur_L + 15) >> 4) - 1;
    valu_write_piece<D, VG>(p, sk, acc, cur_s, cur_kvh, whole, rg.w, lane);
  };

  for (int base = rg.T0; base < rg.T1; base += 64) {
    const int m = min(64, rg.T1 - base);
    const TileMeta meta = fetch_meta<BS>(p, ps, H, base + lane, lane < m);
    auto load = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
      const int jj = min(j, m - 1);
      const Uniform u = read_meta(meta, jj);
      load_tile<D, BS>(p, u.hg, u.b0, u.b1, 16 * u.t, u.L, j < m, lo, kt, vt);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
      const Uniform u = read_meta(meta, j);
      if (u.t == 0 || base + j == rg.T0) {  // a new pair: its q is loaded here (rare)
        if (cur_s >= 0) finish();
        valu_reset(acc);
        valu_load_q<D, VG>(p, u.s, u.hg * VG, lane, qf);
        cur_s = u.s;
        cur_kvh = u.hg;
        cur_t0 = u.t;
        cur_L = u.L;
      }
      cur_tlast = u.t;
      valu_tile<D, VG>(acc, qf, p.scale_log2, 16 * u.t, u.L, lane, kt, vt);
    };
    u32x4 ak[NC], av[NC], bk[NC], bv[NC], ck[NC], cv[NC];
    load(0, ak, av);
    load(1, bk, bv);
    for (int j = 0;; j += 3) {
      load(j + 2, ck, cv);
      compute(j, ak, av);
      if (j + 1 >= m) break;
      load(j + 3, ak, av);
      compute(j + 1, bk, bv);
      if (j + 2 >= m) break;
      load(j + 4, bk, bv);
      compute(j + 2, ck, cv);
      if (j + 3 >= m) break;
    }
  }
  finish();
}

// Log-sum-exp combine of n pieces (rows row0 + i * stride, i ascending) for
// dim d: a single pass with a running max, the loads of up to kBatch pieces
// issued together so the kernel pays one memory latency per batch.
constexpr int kCombineBatch = 16;

template <int D>
__device__ __forceinline__ float lse_combine(const float* ml, const float* o, size_t row0,
                                             size_t stride, int n, int d) {
  float M = kNegInf, num = 0.f, den = 0.f;
  for (int i0 = 0; i0 < n; i0 += kCombineBatch) {
    float m[kCombineBatch], l[kCombineBatch], x[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const bool live = i0 + k < n;
      const size_t row = row0 + size_t(live ? i0 + k : 0) * stride;
      m[k] = live ? ml[row * 2] : kNegInf;
      l[k] = live ? ml[row * 2 + 1] : 0.f;
      x[k] = live ? o[row * D + d] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      if (i0 + k < n) {
        const float Mn = fmaxf(M, m[k]);
        const float a = exp2f(M - Mn);
        const float b = l[k] * exp2f(m[k] - Mn);
        num = num * a + b * x[k];
        den = den * a + b;
        M = Mn;
      }
    }
  }
  return num / den;
}

// The first batch of lse_combine's pieces loaded before the piece count is
// known: rows k < cap (cap <= kCombineBatch, rows the workspace holds for
// this output, written or not), so that the loads go out beside the length's
// instead of after it.  lse_combine_from then uses the first n of them.
struct FirstPieces {
  float m[kCombineBatch], l[kCombineBatch], x[kCombineBatch];
};

template <int D>
__device__ __forceinline__ FirstPieces lse_first_pieces(const float* ml, const float* o, size_t row0,
                                                        size_t stride, int cap, int d) {
  FirstPieces f;
#pragma unroll
  for (int k = 0; k < kCombineBatch; ++k) {
    f.m[k] = kNegInf;
    f.l[k] = 0.f;
    f.x[k] = 0.f;
    if (k < cap) {  // uniform: rows past cap are not loaded (cap 0: no workspace, nothing read)
      const size_t row = row0 + size_t(k) * stride;
      f.m[k] = ml[row * 2];
      f.l[k] = ml[row * 2 + 1];
      f.x[k] = o[row * D + d];
    }
  }
  return f;
}

template <int D>
__device__ __forceinline__ float lse_combine_from(const FirstPieces& f, const float* ml, const float* o,
                                                  size_t row0, size_t stride, int n, int d) {
  float M = kNegInf, num = 0.f, den = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineBatch; ++k) {
    if (k < n) {
      const float Mn = fmaxf(M, f.m[k]);
      const float a = exp2f(M - Mn);
      const float b = f.l[k] * exp2f(f.m[k] - Mn);
      num = num * a + b * f.x[k];
      den = den * a + b;
      M = Mn;
    }
  }
  for (int i0 = kCombineBatch; i0 < n; i0 += kCombineBatch) {
    float m[kCombineBatch], l[kCombineBatch], x[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const bool live = i0 + k < n;
      const size_t row = row0 + size_t(live ? i0 + k : 0) * stride;
      m[k] = live ? ml[row * 2] : kNegInf;
      l[k] = live ? ml[row * 2 + 1] : 0.f;
      x[k] = live ? o[row * D + d] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      if (i0 + k < n) {
        const float Mn = fmaxf(M, m[k]);
        const float a = exp2f(M - Mn);
        const float b = l[k] * exp2f(m[k] - Mn);
        num = num * a + b * x[k];
        den = den * a + b;
        M = Mn;
      }
    }
  }
  return num / den;
}

// Combine the pieces of every pair cut between waves, and write zeros for
// empty contexts.  One workgroup per (sequence, head group) pair.
template <int D>
__global__ __launch_bounds__(512) void combine_sk(DecodeParams p, StreamParams sk) {
  const int H = p.num_kv_heads * p.head_groups;
  const int pair = blockIdx.x;
  const int s = pair / H;
  const int hg = pair - s * H;
  int kvh, h0, ncols;
  head_span(p, hg, kvh, h0, ncols);
  const int* ps = sk.plan + kPlanHeader;
  const int n = ps[s + 1] - ps[s];
  if (n == 0) {
    for (int idx = threadIdx.x; idx < ncols * D; idx += blockDim.x)
      store_out(p, s, h0 + idx / D, idx % D, 0.f);
    return;
  }
  const int per = sk.plan[0];
  const int first = H * ps[s] + hg * n;
  const int wa = first / per;
  const int wb = (first + n - 1) / per;
  if (wa == wb) return;  // one wave saw the whole pair and wrote it
  for (int idx = threadIdx.x; idx < ncols * D; idx += blockDim.x) {
    const int col = idx / D;
    const int d = idx - col * D;
    const float r = lse_combine<D>(sk.ws_ml, sk.ws_o, piece_row(pair, wa, col), 16, wb - wa + 1, d);
    store_out(p, s, h0 + col, d, r);
  }
}

// ===========================================================================
// partitioned schedule
// ===========================================================================

// Block-table entries of up to 64 consecutive tiles of one wave, one per lane,
// so the tile loop never waits on memory for an address: lane j holds the
// entry (entries, for B = 8) of the wave's tile k0 + j.  The load depends
// only on the tile index, not on the context length, so it can be issued
// before the length arrives; it is bounded by the table row, and an entry of
// a tile past the context is never used as an address.
struct TableCache {
  int e0, e1;
};

// Read-only view of row s of the block table (W entries).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t table_row(const DecodeParams& p, int s, int BS) {
  return make_rsrc(p.block_tables + size_t(s) * p.bt_s, (p.max_len / BS) * 4);
}

__device__ __forceinline__ int load_i32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0);
}

template <int BS>
__device__ __forceinline__ TableCache fetch_table(__amdgpu_buffer_rsrc_t row, int tile0, int wave,
                                                  int k0, int lane) {
  const uint32_t t = uint32_t(tile0 + wave + kWaves * (k0 + lane));
  TableCache c{0, 0};
  if constexpr (BS == 16) {
    c.e0 = load_i32(row, t * 4);
  } else if constexpr (BS == 32) {
    c.e0 = load_i32(row, (t >> 1) * 4);
  } else {
    c.e0 = load_i32(row, t * 8);
    c.e1 = load_i32(row, t * 8 + 4);
  }
  return c;
}

// Register slots of the tile pipeline: the tile being computed and one whose
// loads are in flight.  That is enough once every compute unit runs a
// workgroup or more: the memory system is saturated and further loads only
// queue (three or four slots measured no faster), while the registers they
// take keep a third workgroup off each compute unit.  Smaller grids, with a
// wave or two per compute unit, are latency-bound and take kDeepSlots.
constexpr int kPipeSlots = 2;
constexpr int kDeepSlots = 4;

// Walk this wave's tiles (tiles wave, wave + 4, ... of the partition [t0, t1))
// with the next S - 1 tiles' loads issued before the current one is
// computed.  `first` holds the table entries of the wave's first 64 tiles.
struct NoHook {
  __device__ void operator()() const {}
};

template <int D, int BS, int S, typename F, typename H = NoHook>
__device__ __forceinline__ void walk_tiles(const DecodeParams& p, __amdgpu_buffer_rsrc_t row,
                                           TableCache first, int kvh, int t0, int t1, int wave,
                                           int lane, F&& compute, H&& after_first_loads = H{}) {
  constexpr int NC = D / 32;
  const int ntiles = (t1 - t0 + 15) >> 4;
  const int n = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const LaneOffsets<D, BS> lo = lane_offsets<D, BS>(lane);
  // tiles per table fetch: a whole number of rounds, so that only the last
  // chunk has padding tiles, and those lie past the context
  constexpr int kChunk = 64 / S * S;
  TableCache tc = first;
  int k0 = 0;
  int m = min(kChunk, n);
  auto start = [&](int j) { return t0 + 16 * (wave + kWaves * (k0 + j)); };
  auto load = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    const int jj = min(j, m - 1);
    const int b0 = __builtin_amdgcn_readlane(tc.e0, jj);
    int b1 = 0;
    if constexpr (BS == 8) {
      // the second block of a tile whose tokens all lie in the first is not
      // in the table: read the first again (its tokens are masked)
      b1 = __builtin_amdgcn_readlane(tc.e1, jj);
      b1 = start(jj) + 8 < t1 ? b1 : b0;
    }
    load_tile<D, BS>(p, kvh, b0, b1, start(jj), t1, j < m, lo, kt, vt);
    __builtin_amdgcn_sched_barrier(0);
  };
  u32x4 kk[S][NC], vv[S][NC];
  // The first chunk's first loads sit ahead of the chunk loop, in straight
  // code, so that they wait for the table entries alone, not for loads the
  // caller issued after the table's (in-order counter); then the hook.
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i) load(i, kk[i], vv[i]);
  }
  after_first_loads();
  for (; k0 < n; k0 += kChunk) {
    if (k0 > 0) {
      tc = fetch_table<BS>(row, t0 >> 4, wave, k0, lane);
      m = min(kChunk, n - k0);
#pragma unroll
      for (int i = 0; i < S - 1; ++i) load(i, kk[i], vv[i]);
    }
    // The trip count is rounded up to whole rounds of S tiles: the extra tiles
    // lie past t1 (only the last chunk is short), load as zeros without
    // touching memory and add nothing.  A
    // loop that leaves only at the end of a round reaches its head in the same
    // state from both edges, so the compiler waits only for the tile it uses
    // and keeps S - 1 tiles' loads in flight throughout.
    const int rounds = (m + S - 1) / S;
    for (int j = 0; j < rounds * S; j += S) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        load(j + i + S - 1, kk[(i + S - 1) % S], vv[(i + S - 1) % S]);
        compute(start(j + i), kk[i], vv[i]);
      }
    }
  }
}

// Per-workgroup LDS for the cross-wave combine.
template <int D>
struct Smem {
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][D][17];
  float f[kWaves][16];  // column_weights: wave w's weight of column g
  float fn[16];         // column_weights: weight of the folded-in new token of column g
  float M[16];          // column_weights: reference max and sum of column g
  float L[16];
};

// After the waves' (m, l, o) are in sm and a barrier: per column g < ncols,
// the reference max M over the waves, the sum L, and each wave's weight
// 2^(m_w - M) / L (zero where the column saw no token), so that an output
// element is a four-term dot product of sm.o and sm.f.  With xn, column g
// also takes one more token of score xn[g] (log2 units; -inf: none), whose
// value then enters with weight sm.fn[g].  Ends with a barrier.
template <int D>
__device__ __forceinline__ void column_weights(Smem<D>& sm, int ncols, const float* xn = nullptr) {
  if (int(threadIdx.x) < ncols) {
    const int g = threadIdx.x;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][g]);
    float e[kWaves], l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      e[w] = M != kNegInf ? exp2f(sm.m[w][g] - M) : 0.f;
      l += sm.l[w][g] * e[w];
    }
    float a = 1.f, b = 0.f;
    if (xn && xn[g] != kNegInf) {
      const float M2 = fmaxf(M, xn[g]);
      a = exp2f(M - M2);  // 0 where the waves read no token (M = -inf)
      b = exp2f(xn[g] - M2);
      l = l * a + b;
      M = M2;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sm.f[w][g] = e[w] * a * inv;
    sm.fn[g] = b * inv;
    sm.M[g] = M;
    sm.L[g] = l;
  }
  __syncthreads();
}

// Output element (d, column g): the waves' o weighted by column_weights.
template <int D>
__device__ __forceinline__ float weighted_o(const Smem<D>& sm, int d, int g) {
  float o = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) o = fmaf(sm.o[w][d][g], sm.f[w][g], o);
  return o;
}

// Combine the waves' (m, l, o) and write either the output (one partition)
// or this partition's partial result for the combine kernel.
template <int D>
__device__ __forceinline__ void finish_partition(const DecodeParams& p, Smem<D>& sm, int s, int h0,
                                                 int ncols, int part, int nparts) {
  __syncthreads();
  column_weights<D>(sm, ncols);
  if (nparts <= 1) {  // the output, eight dims per thread
    for (int idx = threadIdx.x; idx < ncols * (D / 8); idx += kThreads) {
      const int g = idx / (D / 8);
      const int d0 = 8 * (idx - g * (D / 8));
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = weighted_o<D>(sm, d0 + j, g);
      store_out8(p, s, h0 + g, d0, o);
    }
    return;
  }
  for (int idx = threadIdx.x; idx < ncols * D; idx += kThreads) {  // this partition's piece
    const int g = idx / D;
    const int d = idx - g * D;
    const size_t row = (size_t(s) * p.num_q_heads + h0 + g) * p.max_parts + part;
    p.ws_o[row * D + d] = weighted_o<D>(sm, d, g);
    if (d == 0) {
      p.ws_ml[row * 2 + 0] = sm.M[g];
      p.ws_ml[row * 2 + 1] = sm.L[g];
    }
  }
}

// Sequence that row y of a partitioned grid works on, by rank of its context
// length (rank 0 = longest, ties in index order).  Rows are dispatched in
// order.  When the grid is larger than what the machine holds at once, row y
// takes rank y: the longest contexts start first and the short ones fill the
// machine at the end.  When the whole grid is resident, each compute unit
// receives one workgroup from the rows below p.rank_split and one from the
// rows after it, and the hardware serves the first ahead of the second; the
// rows below the split take the longest contexts in order and the rows after
// it take the rest from the shortest up, so that every compute unit pairs a
// long context with a short one and all finish at about the same time.
// Every workgroup derives the same bijection from the lengths alone.  The rank of a sequence is the
// number of larger keys (length << 9 | 511 - index, unique).  Grids split into
// partitions keep the identity order: there the work of a row is bounded by
// the partition, and neighbouring sequences, which often share prefix blocks
// (parallel samples of one prompt), stay close in time so that the shared
// blocks are still cached when the next one reads them.  So do batches of
// more than kMaxDeviceRanked sequences or with table spans of 2^22 tokens or
// more, unless the host ranked them (has_order 1).
__device__ __forceinline__ int ranked_seq(const DecodeParams& p, int y) {
  const int S = p.num_seqs;
  if (p.has_order == 1) {  // ranked on the host: no round trip to the lengths
    // a 32-bit read at a workgroup-uniform index: a scalar load
    const uint32_t w = reinterpret_cast<const uint32_t*>(p.order)[y >> 1];
    return int((y & 1) ? w >> 16 : w & 0xffffu);
  }
  if (p.max_parts > 1 || S > kMaxDeviceRanked || p.max_len >= (1 << 22)) return y;
  __shared__ uint32_t keys[kMaxDeviceRanked];
  __shared__ int pick;
  const int S16 = (S + 15) & ~15;  // zero keys pad to whole 16-key steps
  for (int u = threadIdx.x; u < S16; u += blockDim.x)
    keys[u] = u < S ? (uint32_t(clamp_len(p, p.context_lens[u])) << 9) | uint32_t(511 - u) : 0u;
  __syncthreads();
  for (int c = threadIdx.x; c < S; c += blockDim.x) {
    const uint32_t kc = keys[c];
    int rank = 0;
    for (int u = 0; u < S16; u += 16) {
      u32x4 k4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) k4[i] = *reinterpret_cast<const u32x4*>(&keys[u + 4 * i]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rank += int(k4[i].x > kc) + int(k4[i].y > kc) + int(k4[i].z > kc) + int(k4[i].w > kc);
    }
    const int row = rank < p.rank_split ? rank : S - 1 - (rank - p.rank_split);
    if (row == y) pick = c;
  }
  __syncthreads();
  return pick;
}

// The waves' MFMA accumulators of one (sequence, head group) through LDS to the
// output or to this partition's partial result.
template <int D>
__device__ __forceinline__ void mfma_finish(const DecodeParams& p, Smem<D>& sm, const MfmaAcc<D>& acc,
                                            int s, int h0, int ncols, int part, int nparts, int wave,
                                            int lane) {
  const int r = lane & 15;
  const int g4 = lane >> 4;
  // column totals over the four 16-lane groups
  float l = acc.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (g4 == 0) {
    sm.m[wave][r] = acc.m;
    sm.l[wave][r] = l;
  }
  if (r < ncols) {  // columns past the group hold nothing
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.o[wave][2 * (4 * g4 + j) + 32 * (mm >> 1) + (mm & 1)][r] = acc.o[mm][j];
  }
  finish_partition<D>(p, sm, s, h0, ncols, part, nparts);
}

// Partitions of a multi-token sequence with L_old cached tokens: the new
// tokens join the last (at least one partition, also with nothing cached).
__device__ __forceinline__ int multi_parts(const DecodeParams& p, int L_old) {
  return max(1, min((L_old + p.part_tokens - 1) / p.part_tokens, p.max_parts));
}

// Partitions of sequence s that this launch covers (clamping keeps the
// partition count consistent with the grid for over-long contexts).
__device__ __forceinline__ int partitions(const DecodeParams& p, int L) {
  return min((clamp_len(p, L) + p.part_tokens - 1) / p.part_tokens, p.max_parts);
}

// SL pipeline slots; the deep pipeline runs where grids hold at most one
// workgroup per compute unit, so it may take the registers of two.
template <int D, int BS, int SL>
__global__ __launch_bounds__(kThreads, (SL == kPipeSlots ? 2 : 1)) void decode_mfma(DecodeParams p) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int hg = blockIdx.x;
  const int s = ranked_seq(p, blockIdx.y);
  const int part = blockIdx.z;
  int kvh, h0, ncols;
  head_span(p, hg, kvh, h0, ncols);
  const int t0 = part * p.part_tokens;
  const auto row = table_row(p, s, BS);
  const TableCache first = fetch_table<BS>(row, t0 >> 4, wave, 0, lane);

  const int L = clamp_len(p, p.context_lens[s]);
  const int nparts = partitions(p, L);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int t1 = min(L, t0 + p.part_tokens);

  u32x4 q[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    q[c] = u32x4{0u, 0u, 0u, 0u};
    if (r < ncols) q[c] = load16(p.q + size_t(s) * p.q_s + size_t(h0 + r) * p.q_h + 8 * (g4 + 4 * c));
  }
  MfmaAcc<D> acc;
  mfma_reset(acc);
  walk_tiles<D, BS, SL>(p, row, first, kvh, t0, t1, wave, lane,
                                             [&](int ts, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    mfma_tile<D>(acc, q, p.scale_log2, ts, t1, lane, kt, vt);
  });

  mfma_finish<D>(p, sm, acc, s, h0, ncols, part, nparts, wave, lane);
}

// Dims 8*piece .. +7 of one token's K and V (kv, vv) into slot `slot` of head h.
template <int D, int BS>
__device__ __forceinline__ void write_slot_piece(uint16_t* k_cache, uint16_t* v_cache, int num_kv_heads,
                                                 int64_t slot, int h, int piece, u32x4 kv, u32x4 vv) {
  const int64_t blk = slot / BS;
  const int off = int(slot - blk * BS);
  const size_t tile = (size_t(blk) * num_kv_heads + h) * (BS * D);
  store16(k_cache + tile + (piece * BS + off) * 8, kv);
  uint16_t* vt = v_cache + tile + ((off >> 2) * D + piece * 8) * 4 + (off & 3);
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vt[(2 * e) * 4] = uint16_t(w[e] & 0xffffu);
    vt[(2 * e + 1) * 4] = uint16_t(w[e] >> 16);
  }
}

// ---------------------------------------------------------------------------
// shared partitions (partitioned schedule, G <= 16)
//
// Sequences that share a prefix hold the same physical blocks for it.  Inside
// an aligned window of 16/G consecutive sequences (the columns of one
// workgroup), a run of sequences whose tables for partition j begin with the
// same blocks is computed by the workgroup of its first sequence, the leader:
// its MFMA columns are (member, query head) pairs, member i's column i*G + g
// holding sequence s+i's query head kvh*G + g.  The tiles the members have in
// common are read once for all columns; then each member's own tiles of the
// partition (a copy-on-write block and what the member wrote since, say) are
// read once, counting for that member's columns only.  The other members'
// workgroups skip partition j.  A run grows only while the members' own tiles
// together stay within the common ones, so a leader reads at most twice a
// partition's tiles.  Every workgroup of the window derives the same runs from
// the same table entries and lengths.  Each member's partial result goes
// where its own workgroup would have put it, and the combine kernel is
// unchanged.
//
// Fused (a decode step, one new token per sequence, in mp's k_new / v_new /
// slots): a sequence's last token, in its last partition, is the new one and
// is not in the pools yet.  The walk reads a member's pool tokens up to it,
// and the new token is folded in from k_new / v_new when the waves are
// joined; combine_append stores it in the pools afterwards (no workgroup of
// this kernel reads its slot), so the step needs no append launch before the
// decode, and no attention workgroup waits at its end for store
// acknowledgements while the reads saturate the memory.
// ---------------------------------------------------------------------------
constexpr int kMaxShare = 16;  // members per workgroup at G = 1

// Over each row of 16 lanes (DPP row shifts; a lane whose source would lie
// before its row takes the identity): the value of the lane before, and the
// inclusive prefix minimum and sum.
__device__ __forceinline__ int row_shift1(int x) { return __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false); }

__device__ __forceinline__ int row_scan_min(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  return x;
}

__device__ __forceinline__ int row_scan_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  return x;
}

// Sequence of grid row y in decode_shared.  An unsplit grid padded to whole
// windows (rows = windows * M, M members each) takes row y as member slot
// j = y / windows of window y % windows, the slots in bit-reversed order when
// M is a power of two: 0, M/2, M/4, 3M/4, ...  A window's runs start at its
// first member and, for runs of 2, 4 or 8 parallel samples, at the multiples
// of the run length, so the run leaders are dispatched ahead of the
// followers, which only plan and leave, and the leaders of all windows start
// together; the followers then take the slots the leaders leave free.  Rows
// past the last sequence return -1.  Split grids keep the identity order:
// there a partition's followers, queued behind its leaders, would hold back
// the next partition's workgroups.
__device__ __forceinline__ int shared_seq(int y, int M, int S) {
  const int windows = (S + M - 1) / M;
  if (gridDim.z != 1 || int(gridDim.y) != windows * M) return y;
  const int j = y / windows;
  int si = j;
  if (M > 1 && (M & (M - 1)) == 0) si = int(__builtin_bitreverse32(uint32_t(j)) >> (32 - __builtin_ctz(M)));
  const int s = (y - j * windows) * M + si;
  return s < S ? s : -1;
}

// Walk a run's nv tiles, tiles wave, wave + 4, ... of it in this wave, with
// the next S - 1 tiles' loads issued before the current one is computed (as
// walk_tiles).  Tiles [0, n_sh) are the common tokens [t0, sh_end) of every
// member, whose block-table entries come from the leader's row (`first`
// holds the wave's first 64, fetched before the plan was known).  The rest are
// the members' own tokens: member c's [t_sh, tw[c]) are tiles n_sh + off[c] ..
// n_sh + off[c+1] - 1, read from its own row; a lane holding one of them
// replaces its entries with the member's and keeps the tile's token range
// (relative to t0, 16 bits each) and member.
template <int D, int BS, int S, typename F>
__device__ __forceinline__ void walk_run(const DecodeParams& p, __amdgpu_buffer_rsrc_t row, TableCache first,
                                         int s, int kvh, int t0, int sh_end, int n_sh, int t_sh, const int* tw,
                                         const int* off, int nv, int wave, int lane, F&& compute) {
  constexpr int NC = D / 32;
  const int n = nv > wave ? (nv - wave + kWaves - 1) / kWaves : 0;
  const LaneOffsets<D, BS> lo = lane_offsets<D, BS>(lane);
  constexpr int kChunk = 64 / S * S;
  for (int k0 = 0; k0 < n; k0 += kChunk) {
    TableCache tc = k0 == 0 ? first : fetch_table<BS>(row, t0 >> 4, wave, k0, lane);
    int range = 0, member = -2;
    {
      const int v = wave + kWaves * (k0 + lane);
      if (v >= n_sh && v < nv) {
        const int w = v - n_sh;
        int c = 0;
        while (off[c + 1] <= w) ++c;
        const int ts = t_sh + 16 * (w - off[c]);
        const int te = tw[c];
        // entries read lie before the member's context end: inside its table row
        const int32_t* own = p.block_tables + size_t(s + c) * p.bt_s;
        if constexpr (BS == 16) {
          tc.e0 = own[ts >> 4];
        } else if constexpr (BS == 32) {
          tc.e0 = own[ts >> 5];
        } else {
          tc.e0 = own[ts >> 3];
          tc.e1 = ts + 8 < te ? own[(ts >> 3) + 1] : tc.e0;
        }
        range = int((uint32_t(te - t0) << 16) | uint32_t(ts - t0));  // both <= 32768: 16 bits each
        member = c;
      }
    }
    const int m = min(kChunk, n - k0);
    // tile j of the chunk (uniform): blocks, first token, mask end, member;
    // selects rather than branches, so the tile loop stays one block
    auto meta = [&](int j, int& b0, int& b1, int& ts, int& te, int& mem) {
      const int v = wave + kWaves * (k0 + j);
      const bool common = v < n_sh;
      const int rg = __builtin_amdgcn_readlane(range, j);
      ts = common ? t0 + 16 * v : t0 + (rg & 0xffff);
      te = common ? sh_end : t0 + int(uint32_t(rg) >> 16);
      mem = common ? -1 : __builtin_amdgcn_readlane(member, j);
      b0 = __builtin_amdgcn_readlane(tc.e0, j);
      b1 = 0;
      if constexpr (BS == 8) {
        const int e1 = __builtin_amdgcn_readlane(tc.e1, j);
        b1 = common && ts + 8 >= te ? b0 : e1;
      }
    };
    auto load = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
      int b0, b1, ts, te, mem;
      meta(min(j, m - 1), b0, b1, ts, te, mem);
      load_tile<D, BS>(p, kvh, b0, b1, ts, te, j < m, lo, kt, vt);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto tile = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
      int b0, b1, ts, te, mem;
      meta(min(j, m - 1), b0, b1, ts, te, mem);
      compute(ts, te, j < m ? mem : -2, kt, vt);  // padding counts for no column
    };
    // whole rounds of S tiles; the padding tiles (past the run) load zeros
    // without touching memory
    const int rounds = (m + S - 1) / S;
    u32x4 kk[S][NC], vv[S][NC];
#pragma unroll
    for (int i = 0; i < S - 1; ++i) load(i, kk[i], vv[i]);
    for (int j = 0; j < rounds * S; j += S) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        load(j + i + S - 1, kk[(i + S - 1) % S], vv[(i + S - 1) % S]);
        tile(j + i, kk[i], vv[i]);
      }
    }
  }
}

template <int D, int BS, bool Fused>
__global__ __launch_bounds__(kThreads, 2) void decode_shared(MultiParams mp) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;
  __shared__ int win_len[kMaxShare];      // window member i: clamped context length
  __shared__ int win_tw[kMaxShare];       // window member i: end of its pool tokens read in this partition
  __shared__ int run_off[kMaxShare + 1];  // leader: first own tile of each member, after the common ones
  __shared__ float x_new[16];             // fused: the new tokens' scores (log2 units), by column
  __shared__ u32x4 v_fold[kMaxShare][D / 8];  // fused: member i's new value, loaded ahead of any store
  const DecodeParams& p = mp.d;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int kvh = blockIdx.x;
  const int part = blockIdx.z;
  const int G = p.group;
  const int M = 16 / G;  // members one workgroup carries
  const int s = shared_seq(blockIdx.y, M, p.num_seqs);
  if (s < 0) return;  // workgroup-uniform: padding of the last window
  const int t0 = part * p.part_tokens;
  const int t_end = t0 + p.part_tokens;
  const int w0 = s - s % M;
  const int si = s - w0;
  const int hi = min(M, p.num_seqs - w0);  // window members present
  const int E0 = t0 / BS;                  // first table entry of the partition (inside the rows)

  // Every load that needs no length first, issued together: this wave's first
  // table entries, and (lanes 0, 1, 2: s-1, s, s+1, or s where there is no
  // such neighbour in the window) the lengths and the partition's first
  // entries of s and its neighbours.  The entry index is kept inside the row;
  // where the partition lies past the table no context reaches it.
  const auto row = table_row(p, s, BS);
  const TableCache first = fetch_table<BS>(row, t0 >> 4, wave, 0, lane);
  const bool has_prev = M > 1 && si > 0, has_next = M > 1 && si + 1 < hi;
  const int last = p.max_len / BS - 1;
  const int nb = lane == 0 && has_prev ? s - 1 : (lane == 2 && has_next ? s + 1 : s);
  const int nb_len = p.context_lens[nb];
  const int nb_ent = p.block_tables[size_t(nb) * p.bt_s + min(E0, last)];
  // Behind those, wave 0 of a workgroup that may share loads what the window
  // plan needs: every member's length (lane i: member i, members past the
  // window repeat the last) and the partition's first 64 entries of every
  // member's row (lane e: entry E0 + e, kept inside the row), so that the
  // plan costs one trip to memory.  A workgroup found alone does not wait for
  // them.  A run's tiles carry 16-bit token offsets inside the partition: at
  // most 32768 tokens.
  const bool may_share = M > 1 && p.part_tokens <= 32768;
  int w_len = 0;
  int w_ent[kMaxShare];
  if (may_share && wave == 0) {
    const int idx = min(E0 + lane, last);
    w_len = p.context_lens[w0 + min(lane, hi - 1)];
#pragma unroll
    for (int i = 0; i < kMaxShare; ++i) w_ent[i] = p.block_tables[size_t(w0 + min(i, hi - 1)) * p.bt_s + idx];
  }
  const int len_prev = __builtin_amdgcn_readlane(nb_len, 0);
  const int len_next = __builtin_amdgcn_readlane(nb_len, 2);
  const int e_prev = __builtin_amdgcn_readlane(nb_ent, 0);
  const int e_self = __builtin_amdgcn_readlane(nb_ent, 1);
  const int e_next = __builtin_amdgcn_readlane(nb_ent, 2);

  const int L = clamp_len(p, __builtin_amdgcn_readlane(nb_len, 1));
  const int nparts = partitions(p, L);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  // the new token of a sequence whose last partition this is (fused step)
  auto owns_new = [&](int len) { return Fused && len > t0 && len <= t_end; };
  // end of the pool tokens this partition holds for a sequence of `len` tokens
  auto pool_end = [&](int len) { return min(len, t_end) - (owns_new(len) ? 1 : 0); };

  // The run this workgroup belongs to (workgroup-uniform).  A run needs a
  // neighbour whose partition starts on the same block; without one (most
  // partitions past a shared prefix) nothing more is read.
  const bool alone = !may_share || L <= t0 ||
                     !((has_prev && clamp_len(p, len_prev) > t0 && e_prev == e_self) ||
                       (has_next && clamp_len(p, len_next) > t0 && e_next == e_self));
  int m = 1, t_sh = 0;
  if (!alone) {
    __shared__ int run_plan[2];  // this workgroup's members (0: a follower) and common end
    if (wave == 0) {
      // member i >= 1 (lane i): the first entry of the partition where its row
      // departs from member i-1's, the lowest set bit of a ballot over the
      // lanes' comparisons, 64 entries a step
      const int E = p.part_tokens / BS;
      int fd_lane = E;
      uint64_t same = 0;  // members whose first 64 entries all match their predecessor's
#pragma unroll
      for (int i = 1; i < kMaxShare; ++i) {
        const uint64_t diff = __ballot(lane < E && w_ent[i] != w_ent[i - 1]);
        if (lane == i && diff) fd_lane = int(__builtin_ctzll(diff));
        if (!diff) same |= uint64_t(1) << i;
      }
      if (E > 64) {  // longer partitions: further chunks for those members
        for (uint64_t u = same & ((uint64_t(1) << hi) - 2); u; u &= u - 1) {
          const int i = int(__builtin_ctzll(u));
          int fd = E;
          for (int c0 = 64; c0 < E; c0 += 64) {
            const int idx = min(E0 + c0 + lane, last);
            const uint64_t diff = __ballot(c0 + lane < E && p.block_tables[size_t(w0 + i) * p.bt_s + idx] !=
                                                                p.block_tables[size_t(w0 + i - 1) * p.bt_s + idx]);
            if (diff) {
              fd = c0 + int(__builtin_ctzll(diff));
              break;
            }
          }
          if (lane == i) fd_lane = fd;
        }
      }
      // pool tokens of each member, and its departure point over the entries
      // both it and its predecessor use (past them the values do not matter)
      auto used = [&](int len) { return len > t0 ? (min(len, t_end) - t0 + BS - 1) / BS : 0; };
      const int my_len = lane < hi ? clamp_len(p, w_len) : 0;
      const int prev_len = row_shift1(my_len);
      const int my_tw = pool_end(my_len);
      const int my_fd = lane > 0 && lane < hi ? min(fd_lane, min(used(my_len), used(prev_len))) : 0;
      if (lane < hi) {
        win_len[lane] = my_len;
        win_tw[lane] = my_tw;
      }
      // Runs from the start of the window, each grown member by member while
      // the members' own tiles stay within the common ones; every workgroup of
      // the window finds the same runs.  For the run from `lead`, lane j takes
      // members lead .. j: their common tiles past t0 (up to the least
      // departure point and pool end) and their own tiles past those (each
      // member's tiles from t0 less the common ones), from prefix scans over
      // the members; the first lane whose member cannot join ends the run.
      const int tiles_from_t0 = (my_tw - t0 + 15) >> 4;
      int lead = 0, mine = 0, mine_tsh = t0;
      for (int it = 0; it < kMaxShare; ++it) {  // each run takes at least one member
        const int mtw = row_scan_min(lane >= lead ? my_tw : INT_MAX);
        const int k = min(E, row_scan_min(lane > lead ? my_fd : INT_MAX));
        const int tiles = row_scan_sum(lane >= lead ? tiles_from_t0 : 0);
        const int common = max(0, min(k * BS, mtw - t0)) >> 4;
        const int own = tiles - (lane - lead + 1) * common;
        const bool stop = lane > lead && lane < hi && (my_tw <= t0 || my_fd == 0 || common == 0 || own > common);
        const uint64_t stops = __ballot(stop);
        const int n = (stops ? int(__builtin_ctzll(stops)) : hi) - lead;
        if (si < lead + n) {
          mine = si == lead ? n : 0;
          mine_tsh = t0 + 16 * (n > 1 ? __builtin_amdgcn_readlane(common, lead + n - 1) : 0);
          break;
        }
        lead += n;
      }
      if (lane == 0) {
        run_plan[0] = mine;
        run_plan[1] = mine_tsh;
      }
    }
    __syncthreads();
    m = __builtin_amdgcn_readfirstlane(run_plan[0]);
    if (m == 0) return;  // the leader computes this partition for s
    t_sh = __builtin_amdgcn_readfirstlane(run_plan[1]);
  }
  const int ncols = m * G;
  // member c's context length (this workgroup's own without a window plan)
  auto member_len = [&](int c) { return m == 1 ? L : win_len[si + c]; };

  // the walk: tokens [t0, sh_end) for every member, then each member's own
  const int sh_end = m > 1 ? t_sh : pool_end(L);
  const int n_sh = sh_end > t0 ? (sh_end - t0 + 15) >> 4 : 0;
  const int* tw = win_tw + si;
  if (m > 1) {
    if (threadIdx.x == 0) {
      int total = 0;
      for (int c = 0; c < m; ++c) {
        run_off[c] = total;
        total += (tw[c] - t_sh + 15) >> 4;
      }
      run_off[m] = total;
    }
    __syncthreads();
  }
  const int nv = __builtin_amdgcn_readfirstlane(n_sh + (m > 1 ? run_off[m] : 0));

  // column r: member r / G, head r % G
  const int ci = r / G;
  const int qh = kvh * G + (r - ci * G);
  u32x4 q[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    q[c] = u32x4{0u, 0u, 0u, 0u};
    if (r < ncols) q[c] = load16(p.q + size_t(s + ci) * p.q_s + size_t(qh) * p.q_h + 8 * (g4 + 4 * c));
  }
  MfmaAcc<D> acc;
  mfma_reset(acc);
  walk_run<D, BS, kPipeSlots>(p, row, first, s, kvh, t0, sh_end, n_sh, t_sh, tw, run_off, nv, wave, lane,
                              [&](int ts, int te, int mem, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    // the tile counts for every column (mem -1), one member's columns, or none
    const int climit = (mem == -1 || mem == ci) ? te - 1 : -1;
    const u32x4 pb = mfma_probs_limit<D>(acc, q, p.scale_log2, ts, climit, lane, kt);
    if (ts + kTileTokens > te) mask_v<D>(vt, ts, te, lane);  // after QK^T: V arrives after K
    mfma_pv<D>(acc, pb, vt);
  });

  if (Fused) {
    // the new tokens' scores for the columns of members whose last partition
    // this is: 16 threads per column, 8 dims each
    const int c = threadIdx.x >> 4;
    const int j = threadIdx.x & 15;
    const int cm = c / G;
    const bool own = c < ncols && owns_new(member_len(cm));
    float dot = 0.f;
    if (own && 8 * j < D) {
      const u32x4 qv = load16(p.q + size_t(s + cm) * p.q_s + size_t(kvh * G + c - cm * G) * p.q_h + 8 * j);
      const u32x4 kv = load16(mp.k_new + size_t(s + cm) * mp.kn_t + size_t(kvh) * mp.kn_h + 8 * j);
      if (c == cm * G) v_fold[cm][j] = load16(mp.v_new + size_t(s + cm) * mp.vn_t + size_t(kvh) * mp.vn_h + 8 * j);
      const uint32_t qa[4] = {qv.x, qv.y, qv.z, qv.w}, ka[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = fmaf(bf_lo(qa[e]), bf_lo(ka[e]), dot);
        dot = fmaf(bf_hi(qa[e]), bf_hi(ka[e]), dot);
      }
    }
    dot += shfl_xor(dot, 1);
    dot += shfl_xor(dot, 2);
    dot += shfl_xor(dot, 4);
    dot += shfl_xor(dot, 8);
    if (j == 0) x_new[c] = own ? dot * p.scale_log2 : kNegInf;
  }

  // combine the waves; column c goes to sequence s + c / G, head kvh * G + c % G
  float l = acc.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (g4 == 0) {
    sm.m[wave][r] = acc.m;
    sm.l[wave][r] = l;
  }
  if (r < ncols) {
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.o[wave][2 * (4 * g4 + j) + 32 * (mm >> 1) + (mm & 1)][r] = acc.o[mm][j];
  }
  __syncthreads();
  column_weights<D>(sm, ncols, Fused ? x_new : nullptr);
  // LDS and registers only from here to the stores: a global load after a
  // store would wait for the store's acknowledgement
  // eight dims per thread, one column's (so one member's) each
  for (int idx = threadIdx.x; idx < ncols * (D / 8); idx += kThreads) {
    const int col = idx / (D / 8);
    const int d0 = 8 * (idx - col * (D / 8));
    const int cm = col / G;
    const int sc = s + cm;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = weighted_o<D>(sm, d0 + j, col);
    if (Fused && sm.fn[col] != 0.f) {  // the new token's value v_new[sc, kvh, d0 .. d0 + 7]
      const u32x4 piece = v_fold[cm][d0 >> 3];
      const uint32_t w[4] = {piece.x, piece.y, piece.z, piece.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = fmaf(sm.fn[col], (j & 1) ? bf_hi(w[j >> 1]) : bf_lo(w[j >> 1]), o[j]);
    }
    const int h = kvh * G + col % G;
    if (partitions(p, member_len(cm)) <= 1) {
      store_out8(p, sc, h, d0, o);
    } else {
      const size_t wrow = (size_t(sc) * p.num_q_heads + h) * p.max_parts + part;
      *reinterpret_cast<f32x4*>(p.ws_o + wrow * D + d0) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(p.ws_o + wrow * D + d0 + 4) = f32x4{o[4], o[5], o[6], o[7]};
      if (d0 == 0) {
        p.ws_ml[wrow * 2 + 0] = sm.M[col];
        p.ws_ml[wrow * 2 + 1] = sm.L[col];
      }
    }
  }
}

template <int D, int BS, int VG>
__global__ __launch_bounds__(kThreads, BS == 8 || VG == 2 ? 1 : 2) void decode_valu(DecodeParams p) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int kvh = blockIdx.x;
  const int s = ranked_seq(p, blockIdx.y);
  const int part = blockIdx.z;
  const int t0 = part * p.part_tokens;
  const auto row = table_row(p, s, BS);
  const TableCache first = fetch_table<BS>(row, t0 >> 4, wave, 0, lane);

  const int L = clamp_len(p, p.context_lens[s]);
  const int nparts = partitions(p, L);
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int t1 = min(L, t0 + p.part_tokens);
  const int h0 = kvh * VG;

  float qf[VG][NC][8];
  valu_load_q<D, VG>(p, s, h0, lane, qf);
  ValuAcc<D, VG> acc;
  valu_reset(acc);
  walk_tiles<D, BS, kPipeSlots>(p, row, first, kvh, t0, t1, wave, lane,
                                                [&](int ts, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    valu_tile<D, VG>(acc, qf, p.scale_log2, ts, t1, lane, kt, vt);
  });

#pragma unroll
  for (int g = 0; g < VG; ++g) {
    float l = acc.l[g];  // per-token shares: sum over the 16 token lanes
    l += shfl_xor(l, 1);
    l += shfl_xor(l, 2);
    l += shfl_xor(l, 4);
    l += shfl_xor(l, 8);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float x = acc.o[g][c][e];  // per-quad shares: sum over the four 16-lane groups
        x += shfl_xor(x, 16);
        x += shfl_xor(x, 32);
        if (g4 == 0) sm.o[wave][2 * r + 32 * c + e][g] = x;
      }
    if (lane == 0) {
      sm.m[wave][g] = acc.m[g];
      sm.l[wave][g] = l;
    }
  }

  finish_partition<D>(p, sm, s, h0, VG, part, nparts);
}

// ---------------------------------------------------------------------------
// contiguous control: the same decode over a cache without paging.  Each
// (sequence, KV head) owns one contiguous run of max_len / 16 tiles, each tile
// in the format of a 16-token block of one head (K [D/8, 16, 8], V [4, D, 4]),
// so the loads are the paged kernel's loads with the tile address computed
// instead of looked up and the tiles of a context adjacent in memory.
// ---------------------------------------------------------------------------
template <int D, int S, typename F>
__device__ __forceinline__ void walk_contiguous(const DecodeParams& p, int s, int kvh, int t1, int wave,
                                                int lane, F&& compute) {
  constexpr int NC = D / 32;
  constexpr int kTileBytes = kTileTokens * D * 2;
  const int ntiles = (t1 + kTileTokens - 1) / kTileTokens;
  const int n = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const int Lmax = p.max_len;
  const size_t region = (size_t(s) * p.num_kv_heads + kvh) * size_t(Lmax) * D;
  const auto rk = make_rsrc(p.k_cache + region, Lmax * D * 2);
  const auto rv = make_rsrc(p.v_cache + region, Lmax * D * 2);
  const auto rz = make_rsrc(p.k_cache, 0);  // zero records: a load through it is free and reads zeros
  const LaneOffsets<D, 16> lo = lane_offsets<D, 16>(lane);
  auto load = [&](int j, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    const bool valid = j < n;
    const auto k_r = valid ? rk : rz;
    const auto v_r = valid ? rv : rz;
    const int toff = valid ? (wave + kWaves * j) * kTileBytes : 0;
    // rows past t1 load zeros, as in the paged walk
    const int ts = kTileTokens * (wave + kWaves * j);
    const uint32_t kx = ts + (lane & 15) >= t1 ? kOutOfRange : 0u;
    const uint32_t vx = ts + 4 * (lane >> 4) >= t1 ? kOutOfRange : 0u;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kt[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            k_r, int((lo.k0 + c * 4 * kTileTokens * 16) | kx), toff, kStreamingLoad));
#pragma unroll
    for (int c = 0; c < NC; ++c)
      vt[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            v_r, int((lo.v0 + c * 256) | vx), toff, kStreamingLoad));
    __builtin_amdgcn_sched_barrier(0);
  };
  const int rounds = (n + S - 1) / S;
  u32x4 kk[S][NC], vv[S][NC];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) load(i, kk[i], vv[i]);
  for (int j = 0; j < rounds * S; j += S) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      load(j + i + S - 1, kk[(i + S - 1) % S], vv[(i + S - 1) % S]);
      compute(kTileTokens * (wave + kWaves * (j + i)), kk[i], vv[i]);
    }
  }
}

template <int D, int SL>
__global__ __launch_bounds__(kThreads, (SL == kPipeSlots ? 2 : 1)) void decode_mfma_contiguous(DecodeParams p) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int s = ranked_seq(p, blockIdx.y);
  int kvh, h0, ncols;
  head_span(p, blockIdx.x, kvh, h0, ncols);
  const int L = clamp_len(p, p.context_lens[s]);
  u32x4 q[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    q[c] = u32x4{0u, 0u, 0u, 0u};
    if (r < ncols) q[c] = load16(p.q + size_t(s) * p.q_s + size_t(h0 + r) * p.q_h + 8 * (g4 + 4 * c));
  }
  MfmaAcc<D> acc;
  mfma_reset(acc);
  walk_contiguous<D, SL>(p, s, kvh, L, wave, lane, [&](int ts, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    mfma_tile<D>(acc, q, p.scale_log2, ts, L, lane, kt, vt);
  });
  mfma_finish<D>(p, sm, acc, s, h0, ncols, 0, 1, wave, lane);
}

// Piece u of a multi-token call's append: row u / (Hkv * D/8), then the head
// and 8 dims.  The row is stored where decode_multi's attention workgroups
// would store it: it lies among the first n of its sequence's rows (n as
// there), and its slot is in the pool (a negative slot skips the store).
template <int D, int BS>
__device__ __forceinline__ void append_piece(const MultiParams& mp, int64_t u) {
  const DecodeParams& p = mp.d;
  const int per_row = p.num_kv_heads * (D / 8);
  const int64_t i64 = u / per_row;
  if (i64 >= mp.num_rows) return;
  const int i = int(i64);
  const int rem = int(u - i64 * per_row);
  const int h = rem / (D / 8);
  const int piece = rem - h * (D / 8);
  // the piece and its slot depend only on the row: their loads go out first
  const int64_t slot = mp.slots[i];
  const u32x4 kv = load16(mp.k_new + size_t(i) * mp.kn_t + size_t(h) * mp.kn_h + piece * 8);
  const u32x4 vv = load16(mp.v_new + size_t(i) * mp.vn_t + size_t(h) * mp.vn_h + piece * 8);
  int s = i, r0 = i, r1 = i + 1;  // no query_start: row s is sequence s's one new token
  if (mp.query_start) {
    // the last sequence whose rows start at or before row i (query_start is
    // non-decreasing), with the kernel's clamping to [0, T)
    auto start = [&](int k) { return min(max(mp.query_start[k], 0), mp.num_rows); };
    if (start(0) > i) return;
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start(mid) <= i) lo = mid; else hi = mid - 1;
    }
    s = lo;
    r0 = start(s);
    r1 = max(start(s + 1), r0);
  } else if (i >= p.num_seqs) {
    return;
  }
  const int n = min(min(r1 - r0, clamp_len(p, p.context_lens[s])), mp.max_query_len);
  if (i - r0 >= n) return;
  if (slot < 0 || slot >= mp.num_slots) return;
  write_slot_piece<D, BS>(mp.k_store, mp.v_store, mp.d.num_kv_heads, slot, h, piece, kv, vv);
}

// ---------------------------------------------------------------------------
// several new tokens per sequence (chunked prefill, speculative verification)
//
// Workgroup (KV head, column group, sequence).  The MFMA columns are (new
// token i, query head g of the group) pairs, column 16 * cg + r = i * G + g,
// so with G * n >= 3 the contraction is real even for MHA.  The cached tokens
// [0, L - n) stream from the pool as in decode; the n new tokens are read from
// k_new / v_new, with token j visible to column (i, g) when j <= i.  The
// column group 0 workgroup of each (sequence, KV head) also appends that
// head's new K/V to their slots; no workgroup reads those slots in this launch.
// ---------------------------------------------------------------------------

// One 16-token tile of new tokens (rows 16u .. 16u + 15 of the sequence's n)
// in the MFMA operand layouts of load_tile; rows past n are zeros.
template <int D>
__device__ __forceinline__ void load_new_tile(const MultiParams& p, int r0, int n, int u, int kvh, int lane,
                                              u32x4 (&kt)[D / 32], u32x4 (&vt)[D / 32]) {
  constexpr int NC = D / 32;
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int jk = 16 * u + r;  // K row of this lane
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    kt[c] = u32x4{0u, 0u, 0u, 0u};
    if (jk < n) kt[c] = load16(p.k_new + size_t(r0 + jk) * p.kn_t + size_t(kvh) * p.kn_h + 8 * (g4 + 4 * c));
  }
  // V: dims 2r + 32c and +1 of tokens 16u + 4*g4 .. +3, packed as (token pair) per dim
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = 16 * u + 4 * g4 + t;
      w[t] = 0u;
      if (j < n)
        w[t] = *reinterpret_cast<const uint32_t*>(p.v_new + size_t(r0 + j) * p.vn_t + size_t(kvh) * p.vn_h +
                                                  2 * r + 32 * c);
    }
    vt[c].x = (w[0] & 0xffffu) | (w[1] << 16);
    vt[c].y = (w[2] & 0xffffu) | (w[3] << 16);
    vt[c].z = (w[0] >> 16) | (w[1] & 0xffff0000u);
    vt[c].w = (w[2] >> 16) | (w[3] & 0xffff0000u);
  }
}

// The same tile (n <= 16 new tokens) from the pieces the append duty parks
// in LDS: piece i * D/8 + j holds dims 8j .. 8j + 7 of new token i.
template <int D>
__device__ __forceinline__ void parked_new_tile(const u32x4* pk, const u32x4* pv, int n, int lane,
                                                u32x4 (&kt)[D / 32], u32x4 (&vt)[D / 32]) {
  constexpr int NC = D / 32;
  constexpr int P = D / 8;
  const int r = lane & 15;
  const int g4 = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c) kt[c] = r < n ? pk[r * P + g4 + 4 * c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = 4 * g4 + t;  // dims 2r + 32c and +1: piece r / 4 + 4c, 32-bit word r % 4
      w[t] = j < n ? reinterpret_cast<const uint32_t*>(&pv[j * P + (r >> 2) + 4 * c])[r & 3] : 0u;
    }
    vt[c].x = (w[0] & 0xffffu) | (w[1] << 16);
    vt[c].y = (w[2] & 0xffffu) | (w[3] << 16);
    vt[c].z = (w[0] >> 16) | (w[1] & 0xffff0000u);
    vt[c].w = (w[2] >> 16) | (w[3] & 0xffff0000u);
  }
}

// A workgroup computes NS sets of 16 columns against each tile it loads, so
// a (sequence, KV head) with up to 16 * NS columns reads its context once.
// Split: the cached context is cut into partitions (grid z), whose pieces the
// combine kernel joins; the unsplit kernel carries none of that (at D = 128,
// B = 16 and one column set its registers leave room for a third workgroup
// per compute unit, which the split kernel's do not).
template <int D, int BS, int NS, bool Split>
__global__ __launch_bounds__(kThreads, (BS == 8 && NS == 2 ? 1 : 2))
void decode_multi(MultiParams mp) {
  constexpr int NC = D / 32;
  __shared__ Smem<D> sm;
  const DecodeParams& p = mp.d;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int kvh = blockIdx.x / mp.col_groups;
  const int cg = blockIdx.x - kvh * mp.col_groups;
  int s, part;
  if constexpr (Split) {
    if (p.has_order == 2) {  // the host's list of (sequence, partition) items
      const int item = p.order[blockIdx.y];
      s = item >> 8;
      part = item & 255;
    } else {
      s = blockIdx.y;
      part = blockIdx.z;
    }
  } else {
    // Grids larger than the GPU holds at once end in rows that only append:
    // the dispatcher starts them last, as slots free up, so that no
    // attention workgroup holds its slot until its stores are acknowledged
    // while the reads still saturate the memory (one-wave grids store at the
    // end of each walk instead).
    if (int(blockIdx.y) >= p.num_seqs) {
      append_piece<D, BS>(mp, (int64_t(blockIdx.y) - p.num_seqs) * gridDim.x * kThreads +
                                  int64_t(blockIdx.x) * kThreads + threadIdx.x);
      return;
    }
    s = ranked_seq(p, blockIdx.y);  // longest contexts first, as decode
    part = 0;
  }
  // This sequence's rows [qa, qb) (no query_start: row s, one new token per
  // sequence), its length and the table entries of the wave's first tiles
  // (they depend only on the sequence and the partition) load together.
  int qa = s, qb = s + 1;
  if (mp.query_start) {
    qa = mp.query_start[s];
    qb = mp.query_start[s + 1];
  }
  const auto row = table_row(p, s, BS);
  const TableCache first = fetch_table<BS>(row, (Split ? part * p.part_tokens : 0) >> 4, wave, 0, lane);
  const int L = clamp_len(p, p.context_lens[s]);
  const int G = p.group;
  // the rows, kept inside [0, T); at most max_query_len of them
  const int r0 = min(max(qa, 0), mp.num_rows);
  const int r1 = min(max(qb, r0), mp.num_rows);
  const int n = min(min(r1 - r0, L), mp.max_query_len);
  const int L_old = L - n;
  // split schedule: partition `part` of the cached tokens; the new tokens
  // belong to the last partition, whose workgroups also append them
  const int nparts = Split ? multi_parts(p, L_old) : 1;
  if (part >= nparts) return;  // workgroup-uniform
  const bool last = part == nparts - 1;
  const int t0 = Split ? part * p.part_tokens : 0;
  const int t1 = Split ? min(L_old, t0 + p.part_tokens) : L_old;

  // The column-group-0 workgroup appends this head's new tokens: its loads
  // go out right after the walk's first tile loads and its pool stores come
  // after the walk, since pool stores ahead of it would hold the walk's pool
  // loads back (loads are not moved across stores that may alias them).  One
  // 16-byte piece per thread here, parked in LDS during the walk (only the
  // thread that loaded a piece reads it back, so no barrier); pieces past the
  // first kThreads are copied at the end.
  __shared__ u32x4 park_k[kThreads], park_v[kThreads];
  __shared__ int64_t park_slot[kThreads];
  const int units = cg == 0 && last && mp.append_rows == 0 ? n * (D / 8) : 0;
  const int staged = min(units, kThreads);
  u32x4 app_k = {0u, 0u, 0u, 0u}, app_v = {0u, 0u, 0u, 0u};
  int64_t app_slot = -1;
  auto load_new = [&]() {
    if (int(threadIdx.x) < staged) {
      const int i = threadIdx.x / (D / 8);
      const int piece = threadIdx.x - i * (D / 8);
      app_slot = mp.slots[r0 + i];
      app_k = load16(mp.k_new + size_t(r0 + i) * mp.kn_t + size_t(kvh) * mp.kn_h + piece * 8);
      app_v = load16(mp.v_new + size_t(r0 + i) * mp.vn_t + size_t(kvh) * mp.vn_h + piece * 8);
    }
  };
  auto append = [&](u32x4 k0, u32x4 v0, int64_t slot0) {
    uint16_t* kc = mp.k_store;
    uint16_t* vc = mp.v_store;
    if (int(threadIdx.x) < staged && slot0 >= 0 && slot0 < mp.num_slots)
      write_slot_piece<D, BS>(kc, vc, p.num_kv_heads, slot0, kvh, threadIdx.x % (D / 8), k0, v0);
    for (int u = threadIdx.x + staged; u < units; u += kThreads) {
      const int i = u / (D / 8);
      const int piece = u - i * (D / 8);
      const int64_t slot = mp.slots[r0 + i];
      if (slot < 0 || slot >= mp.num_slots) continue;
      const u32x4 kv = load16(mp.k_new + size_t(r0 + i) * mp.kn_t + size_t(kvh) * mp.kn_h + piece * 8);
      const u32x4 vv = load16(mp.v_new + size_t(r0 + i) * mp.vn_t + size_t(kvh) * mp.vn_h + piece * 8);
      write_slot_piece<D, BS>(kc, vc, p.num_kv_heads, slot, kvh, piece, kv, vv);
    }
  };
  if (cg == 0 && part == 0) {  // rows past the context (a sequence with no tokens) read as empty: zeros
    const int rows = min(r1 - r0, mp.max_query_len);
    for (int idx = threadIdx.x; idx < (rows - n) * G * D; idx += kThreads) {
      const int i = idx / (G * D);
      const int hd = idx - i * (G * D);
      store_out(p, r0 + n + i, kvh * G + hd / D, hd % D, 0.f);
    }
  }
  const int cols = n * G;             // (query, head) columns of this KV head
  const int col0 = 16 * NS * cg;      // first column of this workgroup
  if (col0 >= cols) {                 // workgroup-uniform; column group 0 only when n == 0
    load_new();
    append(app_k, app_v, app_slot);
    return;
  }

  // column set cs: columns col0 + 16 cs + r; columns past the last query
  // compute with a zero query (never stored) and see every new token
  u32x4 q[NS][NC];
  int qi[NS];
  auto load_q = [&]() {
#pragma unroll
    for (int cs = 0; cs < NS; ++cs) {
      const int c = col0 + 16 * cs + r;
      const bool ok = c < cols;
      qi[cs] = ok ? c / G : n - 1;
      const int qh = kvh * G + (ok ? c - qi[cs] * G : 0);
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        q[cs][k] = u32x4{0u, 0u, 0u, 0u};
        if (ok) q[cs][k] = load16(p.q + size_t(r0 + qi[cs]) * p.q_s + size_t(qh) * p.q_h + 8 * (g4 + 4 * k));
      }
    }
  };
  MfmaAcc<D> acc[NS];
#pragma unroll
  for (int cs = 0; cs < NS; ++cs) mfma_reset(acc[cs]);
  // A single new tile whose pieces are all parked is taken from LDS, first,
  // by the wave the round robin over the waves gives it (the one after the
  // cached tiles' last): its loads then cost no trip to memory at the end of
  // the walk.  The softmax does not depend on the order, up to rounding.
  const int old_tiles = (t1 - t0 + 15) >> 4;
  const bool new_parked = last && n > 0 && n <= kTileTokens && staged == n * (D / 8);  // workgroup-uniform
  // The queries and the new tokens load once each wave's first tile loads
  // are out: ahead of them they would hold those back by a round trip.
  walk_tiles<D, BS, kPipeSlots>(p, row, first, kvh, t0, t1, wave, lane,
                                           [&](int ts, u32x4(&kt)[NC], u32x4(&vt)[NC]) {
    mfma_tile_sets<D, NS>(acc, q, p.scale_log2, ts, t1, lane, kt, vt);
  }, [&]() {
    load_q();
    load_new();
    if (int(threadIdx.x) < staged) {
      park_k[threadIdx.x] = app_k;
      park_v[threadIdx.x] = app_v;
      park_slot[threadIdx.x] = app_slot;
    }
    if (new_parked) {
      __syncthreads();  // every piece parked (every wave comes here once)
      if (wave == old_tiles % kWaves) {
        u32x4 kt[NC], vt[NC];
        parked_new_tile<D>(park_k, park_v, n, lane, kt, vt);
#pragma unroll
        for (int cs = 0; cs < NS; ++cs)
          mfma_tile_causal<D>(acc[cs], q[cs], p.scale_log2, 0, qi[cs], lane, kt, vt);
      }
    }
  });
  // otherwise the new tiles (last partition) continue the cached tiles' round robin over the waves
  for (int u = (wave + kWaves - old_tiles % kWaves) % kWaves; last && !new_parked && 16 * u < n; u += kWaves) {
    u32x4 kt[NC], vt[NC];
    load_new_tile<D>(mp, r0, n, u, kvh, lane, kt, vt);
#pragma unroll
    for (int cs = 0; cs < NS; ++cs)
      mfma_tile_causal<D>(acc[cs], q[cs], p.scale_log2, 16 * u, qi[cs], lane, kt, vt);
  }
  // every pool read of this workgroup is done
  if (int(threadIdx.x) < staged)
    append(park_k[threadIdx.x], park_v[threadIdx.x], park_slot[threadIdx.x]);
  else
    append(app_k, app_v, -1);

  // combine the waves set by set; column (i, g) goes to row r0 + i, head kvh * G + g
#pragma unroll
  for (int cs = 0; cs < NS; ++cs) {
    const int cbase = col0 + 16 * cs;
    const int ncols = min(16, cols - cbase);
    if (ncols <= 0) break;        // workgroup-uniform
    if (cs > 0) __syncthreads();  // the previous set's readers are done with sm
    float l = acc[cs].l;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (g4 == 0) {
      sm.m[wave][r] = acc[cs].m;
      sm.l[wave][r] = l;
    }
    if (r < ncols) {
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sm.o[wave][2 * (4 * g4 + j) + 32 * (mm >> 1) + (mm & 1)][r] = acc[cs].o[mm][j];
    }
    __syncthreads();
    column_weights<D>(sm, ncols);
    if (!Split || nparts <= 1) {  // the output, eight dims per thread
      for (int idx = threadIdx.x; idx < ncols * (D / 8); idx += kThreads) {
        const int col = idx / (D / 8);
        const int d0 = 8 * (idx - col * (D / 8));
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = weighted_o<D>(sm, d0 + j, col);
        const int cc = cbase + col;
        const int i = cc / G;
        store_out8(p, r0 + i, kvh * G + (cc - i * G), d0, o);
      }
    } else {  // this partition's piece of each row for the combine
      for (int idx = threadIdx.x; idx < ncols * D; idx += kThreads) {
        const int col = idx / D;
        const int d = idx - col * D;
        const int cc = cbase + col;
        const int i = cc / G;
        const int h = kvh * G + (cc - i * G);
        const size_t wrow = (size_t(r0 + i) * p.num_q_heads + h) * p.max_parts + part;
        p.ws_o[wrow * D + d] = weighted_o<D>(sm, d, col);
        if (d == 0) {
          p.ws_ml[wrow * 2 + 0] = sm.M[col];
          p.ws_ml[wrow * 2 + 1] = sm.L[col];
        }
      }
    }
  }
}

// Pieces of each new token's row, combined in ascending token order.  One
// thread per (head, dim) of a sequence's row: grid z strides over the rows, so
// that the rows' round trips to the workspace overlap instead of queueing.
template <int D>
__global__ __launch_bounds__(256) void combine_rows(MultiParams mp) {
  const DecodeParams& p = mp.d;
  const int s = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.num_q_heads * D) return;
  int qa = s, qb = s + 1;
  if (mp.query_start) {
    qa = mp.query_start[s];
    qb = mp.query_start[s + 1];
  }
  const int L = clamp_len(p, p.context_lens[s]);
  const int r0 = min(max(qa, 0), mp.num_rows);
  const int r1 = min(max(qb, r0), mp.num_rows);
  const int h = idx / D;
  const int d = idx - h * D;
  // this thread's first row (grid z strides over the rows): its pieces load
  // beside the length's
  const int i0 = blockIdx.z;
  const bool has_first = i0 < min(r1 - r0, mp.max_query_len);
  const size_t first_row0 = (size_t(has_first ? r0 + i0 : 0) * p.num_q_heads + h) * p.max_parts;
  const FirstPieces f = lse_first_pieces<D>(p.ws_ml, p.ws_o, first_row0, 1, (p.ws_ml ? min(p.max_parts, kCombineBatch) : 0), d);
  const int n = min(min(r1 - r0, L), mp.max_query_len);
  const int nparts = multi_parts(p, L - n);
  if (nparts <= 1) return;  // the kernel wrote these rows directly
  if (i0 < n) store_out(p, r0 + i0, h, d, lse_combine_from<D>(f, p.ws_ml, p.ws_o, first_row0, 1, nparts, d));
  for (int i = i0 + gridDim.z; i < n; i += gridDim.z) {
    const size_t row0 = (size_t(r0 + i) * p.num_q_heads + h) * p.max_parts;
    store_out(p, r0 + i, h, d, lse_combine<D>(p.ws_ml, p.ws_o, row0, 1, nparts, d));
  }
}

// Partition combine: one thread per (head, dim) of a sequence.
template <int D>
__global__ __launch_bounds__(256) void combine_parts(DecodeParams p) {
  const int s = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.num_q_heads * D) return;
  const int h = idx / D;
  const int d = idx - h * D;
  const size_t row0 = (size_t(s) * p.num_q_heads + h) * p.max_parts;
  const FirstPieces f = lse_first_pieces<D>(p.ws_ml, p.ws_o, row0, 1, (p.ws_ml ? min(p.max_parts, kCombineBatch) : 0), d);
  const int nparts = partitions(p, p.context_lens[s]);
  if (nparts <= 1) return;  // the decode kernel wrote this row directly
  store_out(p, s, h, d, lse_combine_from<D>(f, p.ws_ml, p.ws_o, row0, 1, nparts, d));
}

// The same combine after decode_shared's fused step, which also stores the
// step's new tokens (one per sequence, from mp's k_new / v_new) at their
// slots: one 16-byte piece of sequence s's token per thread, dealt over all
// workgroups of its row, so that each holds only a few stores.
template <int D, int BS>
__global__ __launch_bounds__(256) void combine_append(MultiParams mp) {
  const DecodeParams& p = mp.d;
  const int s = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int u = threadIdx.x * gridDim.x + blockIdx.x;
  // Every load first, the stores last: a store ahead of a load would hold it
  // back until the store is acknowledged.
  const int64_t slot = mp.slots[s];
  const bool app = u < p.num_kv_heads * (D / 8) && slot >= 0 && slot < mp.num_slots;
  const int ah = u / (D / 8);
  const int piece = u - ah * (D / 8);
  u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
  if (app) {
    kv = load16(mp.k_new + size_t(s) * mp.kn_t + size_t(ah) * mp.kn_h + piece * 8);
    vv = load16(mp.v_new + size_t(s) * mp.vn_t + size_t(ah) * mp.vn_h + piece * 8);
  }
  // rows whose context is split; the decode kernel wrote the others directly
  const int h = idx / D;
  const int d = idx - h * D;
  const bool thread_out = idx < p.num_q_heads * D;
  const size_t row0 = (size_t(s) * p.num_q_heads + (thread_out ? h : 0)) * p.max_parts;
  const FirstPieces f = lse_first_pieces<D>(p.ws_ml, p.ws_o, row0, 1, (p.ws_ml ? min(p.max_parts, kCombineBatch) : 0),
                                            thread_out ? d : 0);
  const int nparts = partitions(p, p.context_lens[s]);
  const bool out = thread_out && nparts > 1;
  float o = 0.f;
  if (out) o = lse_combine_from<D>(f, p.ws_ml, p.ws_o, row0, 1, nparts, d);
  if (app) write_slot_piece<D, BS>(mp.k_store, mp.v_store, p.num_kv_heads, slot, ah, piece, kv, vv);
  if (out) store_out(p, s, h, d, o);
}

// ---------------------------------------------------------------------------
// slot-mapped append
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int i = blockIdx.x;
  const int units = p.num_kv_heads * (D / 8);
  const int u0 = blockIdx.y * blockDim.x + threadIdx.x;
  auto load = [&](int u, u32x4& kv, u32x4& vv) {
    const int h = u / (D / 8);
    const int piece = u - h * (D / 8);
    kv = load16(p.k + size_t(i) * p.k_t + size_t(h) * p.k_h + piece * 8);
    vv = load16(p.v + size_t(i) * p.v_t + size_t(h) * p.v_h + piece * 8);
  };
  // the first piece loads beside the slot, not after it
  const int64_t slot = p.slots[i];
  u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
  if (u0 < units) load(u0, kv, vv);
  if (slot < 0) return;
  for (int u = u0; u < units; u += gridDim.y * blockDim.x) {
    if (u != u0) load(u, kv, vv);
    const int h = u / (D / 8);
    write_slot_piece<D, BS>(p.k_cache, p.v_cache, p.num_kv_heads, slot, h, u - h * (D / 8), kv, vv);
  }
}

// ---------------------------------------------------------------------------
// batched block copy (copy-on-write): every pending copy of a step in one
// launch.  Workgroup (x, y) copies kCopyUnits * 256 16-byte units of one
// pool's block for pair y (the first workgroups of a row take the K pool, the
// rest the V pool), all loads in flight before the stores; a pair naming a
// block outside the pool is skipped.
// ---------------------------------------------------------------------------
constexpr int kCopyUnits = 4;
constexpr int kCopyChunk = kCopyUnits * 256;  // units per workgroup

__global__ __launch_bounds__(256) void copy_kernel(CopyParams p) {
  const size_t block_elems = size_t(p.block_units) * 8;
  const int64_t per_pool = (p.block_units + kCopyChunk - 1) / kCopyChunk;
  const bool is_v = blockIdx.x >= per_pool;
  const int64_t chunk = is_v ? blockIdx.x - per_pool : blockIdx.x;
  uint16_t* const pool = is_v ? p.v_cache : p.k_cache;
  for (int pair = blockIdx.y; pair < p.num_pairs; pair += gridDim.y) {
    const int64_t src = p.pairs[2 * size_t(pair)];
    const int64_t dst = p.pairs[2 * size_t(pair) + 1];
    if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks) continue;
    u32x4 x[kCopyUnits];
#pragma unroll
    for (int i = 0; i < kCopyUnits; ++i) {
      const int64_t u = chunk * kCopyChunk + i * 256 + threadIdx.x;
      const int64_t uu = u < p.block_units ? u : 0;  // in bounds; not stored
      x[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(pool + size_t(src) * block_elems + size_t(uu) * 8));
    }
#pragma unroll
    for (int i = 0; i < kCopyUnits; ++i) {
      const int64_t u = chunk * kCopyChunk + i * 256 + threadIdx.x;
      if (u < p.block_units) store16(pool + size_t(dst) * block_elems + size_t(u) * 8, x[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Name of a kernel instantiation, as pa_last_launch reports it.
std::string kname(const char* fmt, int a = 0, int b = 0, int c = 0) {
  char buf[96];
  snprintf(buf, sizeof(buf), fmt, a, b, c);
  return buf;
}

std::string multi_name(int d, int bs, int ns, bool split) {
  return kname(split ? "decode_multi<%d,%d,%d,true>" : "decode_multi<%d,%d,%d,false>", d, bs, ns);
}

// The status of the launch just made; a successful one is recorded for pa_last_launch.
hipError_t launched(const std::string& name) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) note_launch(name.c_str());
  return e;
}

// The main decode kernel of a call, optionally bracketed by timing events.
template <typename K, typename... A>
hipError_t launch_main(const std::string& name, K kernel, dim3 grid, dim3 block, const LaunchCtx& c, A... args) {
  if (c.start && c.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, c.stream, c.start, c.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, c.stream, args...);
  return launched(name);
}

// Workgroups of a kernel that one compute unit holds at once (its occupancy).
template <typename K>
int resident_per_cu(K kernel) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess || occ < 1)
    occ = 1;
  return occ;
}

// Split row for ranked_seq: the rows whose workgroups the dispatcher places
// first, one per compute unit, when the whole grid fits on the machine at
// once (occ resident workgroups per compute unit); else every row, which is
// plain longest-first.
inline int rank_split_of(const DecodeParams& p, int row_wgs, int occ, const LaunchCtx& c) {
  const int64_t wgs = int64_t(row_wgs) * p.num_seqs;
  if (wgs > int64_t(c.cus) * occ) return p.num_seqs;
  return int(std::min<int64_t>(p.num_seqs, (c.cus + row_wgs - 1) / row_wgs));
}

// The same ranking as ranked_seq's, on the host from a host copy of the
// lengths: clamped length, longest first, equal lengths by index; rows below
// rank_split take the ranks in order, the rest from the shortest up.  The
// order is a permutation whatever the lengths say, so lengths that differ
// from the device's change only the placement, never a result.
inline void fill_order(DecodeParams& p, const LaunchCtx& c) {
  p.has_order = 0;
  const int S = p.num_seqs;
  if (!c.host_lens || p.max_parts > 1 || S > kMaxOrder) return;
  int idx[kMaxOrder];
  for (int i = 0; i < S; ++i) idx[i] = i;
  auto len = [&](int i) { return std::min(std::max(c.host_lens[i], 0), p.max_len); };
  std::stable_sort(idx, idx + S, [&](int a, int b) { return len(a) > len(b); });
  for (int r = 0; r < S; ++r) p.order[r < p.rank_split ? r : S - 1 - (r - p.rank_split)] = uint16_t(idx[r]);
  p.has_order = 1;
}

template <typename K>
hipError_t launch_rows(const std::string& name, K kernel, DecodeParams p, int row_wgs, const LaunchCtx& c) {
  p.rank_split = p.max_parts == 1 ? rank_split_of(p, row_wgs, resident_per_cu(kernel), c) : p.num_seqs;
  fill_order(p, c);
  return launch_main(name, kernel, dim3(row_wgs, p.num_seqs, p.max_parts), dim3(kThreads), c, p);
}

// Fewer MFMA workgroups than compute units: take the deep pipeline.
inline bool deep_pipeline(const DecodeParams& p, const LaunchCtx& c) {
  return int64_t(p.num_kv_heads) * p.head_groups * p.num_seqs * p.max_parts < c.cus;
}

// The shared-partition kernel takes a partitioned schedule of at most 16 q
// heads per KV head whose grid fills the GPU: split on the MFMA path, or
// unsplit with one or two q heads per KV head on the automatic path.
inline bool shared_applies(const DecodeParams& p, Path path, const LaunchCtx& c) {
  return p.group <= 16 && ((path == Path::Mfma && p.max_parts > 1) || (p.share_unsplit && p.max_parts == 1)) &&
         int64_t(p.num_kv_heads) * p.num_seqs * p.max_parts >= c.cus;
}

// Grid rows of decode_shared: unsplit, the sequences padded to whole windows
// of 16 / G members (shared_seq's order) where that stays within the 65535
// rows a grid dimension takes; otherwise exactly the sequences.
inline int shared_rows(const DecodeParams& p) {
  const int M = 16 / p.group;
  const int rows = (p.num_seqs + M - 1) / M * M;
  return p.max_parts == 1 && rows <= 65535 ? rows : p.num_seqs;
}

template <int D, int BS>
hipError_t launch_partitioned(const DecodeParams& p, Path path, const LaunchCtx& c) {
  static_assert(kDeepSlots > kPipeSlots, "");
  hipError_t e;
  if (path == Path::Mfma && deep_pipeline(p, c))
    e = launch_rows(kname("decode_mfma<%d,%d,%d>", D, BS, kDeepSlots), decode_mfma<D, BS, kDeepSlots>, p,
                    p.num_kv_heads * p.head_groups, c);
  else if (shared_applies(p, path, c))
    e = launch_main(kname("decode_shared<%d,%d,false>", D, BS), decode_shared<D, BS, false>,
                    dim3(p.num_kv_heads, shared_rows(p), p.max_parts), dim3(kThreads), c,
                    MultiParams{p});  // split: shared partitions read once (no ranking)
  else if (path == Path::Mfma)
    e = launch_rows(kname("decode_mfma<%d,%d,%d>", D, BS, kPipeSlots), decode_mfma<D, BS, kPipeSlots>, p,
                    p.num_kv_heads * p.head_groups, c);
  else if (p.group == 1)
    e = launch_rows(kname("decode_valu<%d,%d,1>", D, BS), decode_valu<D, BS, 1>, p, p.num_kv_heads, c);
  else
    e = launch_rows(kname("decode_valu<%d,%d,2>", D, BS), decode_valu<D, BS, 2>, p, p.num_kv_heads, c);
  if (e != hipSuccess || p.max_parts <= 1) return e;
  const dim3 cgrid((p.num_q_heads * D + 255) / 256, p.num_seqs);
  hipLaunchKernelGGL((combine_parts<D>), cgrid, dim3(256), 0, c.stream, p);
  return launched(kname("combine_parts<%d>", D));
}

// The partitioned schedule's decode_shared launch with the step's new tokens
// (one per sequence in m) read from k_new / v_new, then the combine, which
// stores them.
template <int D, int BS>
hipError_t launch_shared_step_d(const MultiParams& m, const LaunchCtx& c) {
  const DecodeParams& p = m.d;
  hipError_t e = launch_main(kname("decode_shared<%d,%d,true>", D, BS), decode_shared<D, BS, true>,
                             dim3(p.num_kv_heads, shared_rows(p), p.max_parts), dim3(kThreads), c, m);
  if (e != hipSuccess) return e;
  // num_kv_heads * D / 8 <= num_q_heads * D: the combine's rows cover the pieces
  const dim3 cgrid((p.num_q_heads * D + 255) / 256, p.num_seqs);
  hipLaunchKernelGGL((combine_append<D, BS>), cgrid, dim3(256), 0, c.stream, m);
  return launched(kname("combine_append<%d,%d>", D, BS));
}

// Persistent grid: as many workgroups as can be resident at once (all waves
// stream concurrently; a second round would repeat the start-up latency).
template <typename K>
hipError_t launch_persistent(const std::string& name, K kernel, const DecodeParams& p, const StreamParams& sk,
                             const LaunchCtx& c) {
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0);
  if (e != hipSuccess) return e;
  const int per_cu = std::max(1, std::min(sk.workgroups_per_cu, occ));
  const int wgs = std::min(sk.cus * per_cu, kMaxStreamWaves / kWaves);
  return launch_main(name, kernel, dim3(wgs), dim3(kThreads), c, p, sk);
}

template <int D, int BS>
hipError_t launch_stream(const DecodeParams& p, const StreamParams& sk, Path path, const LaunchCtx& c) {
  hipError_t e;
  if (path == Path::Mfma)
    e = launch_persistent(kname("decode_mfma_sk<%d,%d>", D, BS), decode_mfma_sk<D, BS>, p, sk, c);
  else if (p.group == 1)
    e = launch_persistent(kname("decode_valu_sk<%d,%d,1>", D, BS), decode_valu_sk<D, BS, 1>, p, sk, c);
  else
    e = launch_persistent(kname("decode_valu_sk<%d,%d,2>", D, BS), decode_valu_sk<D, BS, 2>, p, sk, c);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_sk<D>), dim3(p.num_seqs * p.num_kv_heads * p.head_groups), dim3(512), 0,
                     c.stream, p, sk);
  return launched(kname("combine_sk<%d>", D));
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, const StreamParams* sk, int block_size, Path path,
                           const LaunchCtx& c) {
  switch (block_size) {
    case 8: return sk ? launch_stream<D, 8>(p, *sk, path, c) : launch_partitioned<D, 8>(p, path, c);
    case 16: return sk ? launch_stream<D, 16>(p, *sk, path, c) : launch_partitioned<D, 16>(p, path, c);
    case 32: return sk ? launch_stream<D, 32>(p, *sk, path, c) : launch_partitioned<D, 32>(p, path, c);
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
  return launched(kname("append_kernel<%d,%d>", D, block_size));
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const StreamParams* sk, int head_dim, int block_size,
                         Path path, const LaunchCtx& ctx) {
  if (head_dim == 64) return launch_decode_d<64>(p, sk, block_size, path, ctx);
  if (head_dim == 128) return launch_decode_d<128>(p, sk, block_size, path, ctx);
  return hipErrorInvalidValue;
}

bool shared_step_applies(const DecodeParams& p, Path path, const LaunchCtx& c) { return shared_applies(p, path, c); }

hipError_t launch_shared_step(const MultiParams& m, int head_dim, int block_size, const LaunchCtx& c) {
  if (!shared_applies(m.d, Path::Mfma, c)) return hipErrorInvalidValue;
  switch (head_dim * 100 + block_size) {
    case 6408: return launch_shared_step_d<64, 8>(m, c);
    case 6416: return launch_shared_step_d<64, 16>(m, c);
    case 6432: return launch_shared_step_d<64, 32>(m, c);
    case 12808: return launch_shared_step_d<128, 8>(m, c);
    case 12816: return launch_shared_step_d<128, 16>(m, c);
    case 12832: return launch_shared_step_d<128, 32>(m, c);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_contiguous(const DecodeParams& p, int head_dim, const LaunchCtx& ctx) {
  DecodeParams q = p;
  q.max_parts = 1;
  const int row_wgs = p.num_kv_heads * p.head_groups;
  // the pipeline depth the paged kernel takes for the same grid
  const bool deep = deep_pipeline(q, ctx);
  if (head_dim == 64)
    return deep ? launch_rows(kname("decode_mfma_contiguous<64,%d>", kDeepSlots),
                              decode_mfma_contiguous<64, kDeepSlots>, q, row_wgs, ctx)
                : launch_rows(kname("decode_mfma_contiguous<64,%d>", kPipeSlots),
                              decode_mfma_contiguous<64, kPipeSlots>, q, row_wgs, ctx);
  if (head_dim == 128)
    return deep ? launch_rows(kname("decode_mfma_contiguous<128,%d>", kDeepSlots),
                              decode_mfma_contiguous<128, kDeepSlots>, q, row_wgs, ctx)
                : launch_rows(kname("decode_mfma_contiguous<128,%d>", kPipeSlots),
                              decode_mfma_contiguous<128, kPipeSlots>, q, row_wgs, ctx);
  return hipErrorInvalidValue;
}

template <typename K>
hipError_t launch_multi_k(const std::string& name, K kernel, MultiParams p, int head_dim, const LaunchCtx& c) {
  const int row_wgs = p.d.num_kv_heads * p.col_groups;
  if (p.num_items > 0)  // split over the host's (sequence, partition) list
    return launch_main(name, kernel, dim3(row_wgs, p.num_items, 1), dim3(kThreads), c, p);
  const int occ = p.d.max_parts == 1 ? resident_per_cu(kernel) : 1;
  p.d.rank_split = p.d.max_parts == 1 ? rank_split_of(p.d, row_wgs, occ, c) : p.d.num_seqs;
  fill_order(p.d, c);
  // unsplit grids that the GPU cannot hold at once append from rows of their own, started last
  p.append_rows = 0;
  if (p.d.max_parts == 1) {
    if (int64_t(row_wgs) * p.d.num_seqs > int64_t(c.cus) * occ) {
      const int64_t pieces = int64_t(p.num_rows) * p.d.num_kv_heads * (head_dim / 8);
      const int64_t per_row = int64_t(row_wgs) * kThreads;
      const int64_t rows = (pieces + per_row - 1) / per_row;
      if (p.d.num_seqs + rows <= 65535) p.append_rows = int(rows);
    }
  }
  return launch_main(name, kernel, dim3(row_wgs, p.d.num_seqs + p.append_rows, p.d.max_parts), dim3(kThreads), c,
                     p);
}

template <int D, int NS, bool Split>
hipError_t launch_multi_split(const MultiParams& p, int block_size, const LaunchCtx& c) {
  switch (block_size) {
    case 8: return launch_multi_k(multi_name(D, 8, NS, Split), decode_multi<D, 8, NS, Split>, p, D, c);
    case 16: return launch_multi_k(multi_name(D, 16, NS, Split), decode_multi<D, 16, NS, Split>, p, D, c);
    case 32: return launch_multi_k(multi_name(D, 32, NS, Split), decode_multi<D, 32, NS, Split>, p, D, c);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int NS>
hipError_t launch_multi_ns(const MultiParams& p, int block_size, const LaunchCtx& c) {
  return p.d.max_parts > 1 ? launch_multi_split<D, NS, true>(p, block_size, c)
                           : launch_multi_split<D, NS, false>(p, block_size, c);
}

template <int D>
hipError_t launch_multi_d(const MultiParams& p, int block_size, const LaunchCtx& c) {
  const hipError_t e =
      p.col_sets == 1 ? launch_multi_ns<D, 1>(p, block_size, c) : launch_multi_ns<D, 2>(p, block_size, c);
  if (e != hipSuccess || p.d.max_parts <= 1) return e;
  const dim3 cgrid((p.d.num_q_heads * D + 255) / 256, p.d.num_seqs, std::min(p.max_query_len, 65535));
  hipLaunchKernelGGL((combine_rows<D>), cgrid, dim3(256), 0, c.stream, p);
  return launched(kname("combine_rows<%d>", D));
}

hipError_t launch_multi(const MultiParams& p, int head_dim, int block_size, const LaunchCtx& c) {
  if (head_dim == 64) return launch_multi_d<64>(p, block_size, c);
  if (head_dim == 128) return launch_multi_d<128>(p, block_size, c);
  return hipErrorInvalidValue;
}

hipError_t launch_copy(const CopyParams& p, hipStream_t stream) {
  const int64_t gx = 2 * ((p.block_units + kCopyChunk - 1) / kCopyChunk);
  const dim3 grid(unsigned(gx), unsigned(std::min(p.num_pairs, 65535)));
  hipLaunchKernelGGL(copy_kernel, grid, dim3(256), 0, stream, p);
  return launched("copy_kernel");
}

hipError_t launch_append(const AppendParams& p, int head_dim, int block_size, hipStream_t stream) {
  if (head_dim == 64) return launch_append_d<64>(p, block_size, stream);
  if (head_dim == 128) return launch_append_d<128>(p, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
