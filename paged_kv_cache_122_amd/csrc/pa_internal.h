// Internal interface between the host API (pa_api.cpp) and the kernels
// (pa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace pa {

// Tokens per MFMA row tile: every decode kernel walks the context 16 tokens
// at a time (one block at B = 16, half a block at B = 32, two at B = 8).
constexpr int kTileTokens = 16;
constexpr int kWaves = 4;               // waves per decode workgroup
constexpr int kDefaultPartition = 512;  // tokens per partition on the partitioned schedule
// stream-K schedule limits: the per-workgroup tile prefix lives in LDS, and
// partial results are sized for at most this many waves
constexpr int kMaxStreamSeqs = 8192;
// Ordering the rows of an unsplit grid by context length: each workgroup ranks
// up to kMaxDeviceRanked sequences itself (keys in LDS); a host copy of the
// lengths lets the host rank up to kMaxOrder, passed in the kernel arguments
// (the order array keeps every parameter struct within 4 KiB of kernel
// arguments).  Larger batches keep index order.
constexpr int kMaxDeviceRanked = 256;
constexpr int kMaxOrder = 1536;
// The split multi-token grid's (sequence, partition) list: 8 bits each.
constexpr int kMaxItemSeqs = 256;
constexpr int kMaxStreamWaves = 4096;
constexpr int kDefaultWorkgroupsPerCu = 2;
constexpr int kPlanHeader = 4;  // ints before the tile prefix in the stream-K plan

enum class Path : int { Valu = 1, Mfma = 2 };

struct DecodeParams {
  // output [S, Hq, D]: bf16 (out_f32 == 0) or f32
  void* out;
  int64_t out_s, out_h;
  int out_f32;
  // query [S, Hq, D] bf16
  const uint16_t* q;
  int64_t q_s, q_h;
  // pools
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  // block tables [S, W] int32, context lengths [S] int32
  const int32_t* block_tables;
  int64_t bt_s;
  const int32_t* context_lens;
  int num_seqs, num_q_heads, num_kv_heads;
  int group;            // q heads per kv head (G)
  int head_groups;      // ceil(G / 16) column groups per kv head on the MFMA path, 1 on VALU
  int max_len;          // W * B: longer contexts are clamped (a contract violation)
  float scale_log2;     // scale * log2(e)
  // partitioned schedule
  int part_tokens;      // tokens per partition (multiple of 32)
  int max_parts;        // partitions launched per sequence
  int rank_split;       // unsplit grids: rows below it take the longest contexts in
                        // order, the rows from it on the rest from the shortest up
  float* ws_o;          // [S, Hq, max_parts, D]  normalised partial outputs
  float* ws_ml;         // [S, Hq, max_parts, 2]  (reference max in log2 units, sum)
  // has_order 1 (unsplit grids): order[row] is the row's sequence, ranked on
  // the host from a host copy of context_lens (0: ranked by each workgroup).
  // has_order 2 (split multi-token grid): order[y] = sequence << 8 | partition,
  // the grid's rows listing only the partitions that hold tokens.
  int has_order;
  // automatic path, one partition per sequence, 1-2 q heads per KV head: a
  // grid that fills the GPU runs the shared-partition kernel (prefixes that
  // neighbouring sequences share are read once) instead of the VALU kernel
  int share_unsplit;
  uint16_t order[kMaxOrder];
};

// stream-K schedule: plan = {tiles per wave, total tiles, -, -, prefix[S + 1]}
// (written by the decode kernel, read by its combine kernel); partial results
// are indexed by (pair + wave) * 16 + column.
struct StreamParams {
  int* plan;
  float* ws_ml;  // [pieces * 16, 2]
  float* ws_o;   // [pieces * 16, D]
  int cus;              // compute units of the device
  int workgroups_per_cu;  // requested; the launcher caps it at the kernel's occupancy
};

struct AppendParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_t, k_h, v_t, v_h;   // element strides of k, v rows
  const int64_t* slots;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int num_tokens, num_kv_heads;
};

// Several new tokens per sequence in one step: DecodeParams describes q / out
// by row (one row per new token) and the pools, tables and lengths as for
// decode; the new tokens' K/V come from k_new / v_new and are appended.
struct MultiParams {
  DecodeParams d;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t kn_t, kn_h, vn_t, vn_h;  // element strides of k_new, v_new rows
  const int64_t* slots;
  uint16_t* k_store;               // the pools again, written by the append
  uint16_t* v_store;
  const int32_t* query_start;      // [S + 1], or null: row s is sequence s's one new token
  int num_rows;                    // T
  int max_query_len;               // rows per sequence the grid covers
  int col_sets;                    // 16-column MFMA sets per workgroup (1 or 2)
  int col_groups;                  // workgroups per KV head: ceil(max_query_len * G / (16 * col_sets))
  int64_t num_slots;               // num_blocks * block_size
  int num_items;                   // > 0: grid rows from d.order (has_order 2), one partition each
  int append_rows;                 // > 0 (unsplit grids larger than the GPU holds at once): rows
                                   // after the sequences' rows that only append, started last
};

static_assert(sizeof(MultiParams) + sizeof(StreamParams) <= 4096,
              "kernel arguments stay within 4 KiB");
static_assert(offsetof(DecodeParams, order) % 4 == 0 && kMaxOrder % 2 == 0,
              "the order array is read two entries per 32-bit word");

struct CopyParams {
  const int64_t* pairs;  // [N, 2] (src, dst) physical block ids
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t num_blocks;
  int64_t block_units;   // 16-byte units in one block of one pool
  int num_pairs;
};

// Workspace layouts shared by the host planner and the kernels.
struct WorkspaceLayout {
  size_t plan_off, ml_off, o_off, total;
};
WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                                 int64_t max_parts);
WorkspaceLayout stream_workspace_layout(int64_t num_seqs, int64_t num_pairs, int64_t head_dim);

// sk == nullptr: partitioned schedule
// Where a decode is enqueued.  When both events are set, the main decode
// kernel (not the combine) is launched so that they record its own start and
// end (hipExtLaunchKernel).
struct LaunchCtx {
  hipStream_t stream;
  hipEvent_t start;
  hipEvent_t stop;
  int cus;  // compute units of the device
  const int32_t* host_lens = nullptr;  // host copy of context_lens [S], or null
};

hipError_t launch_decode(const DecodeParams& p, const StreamParams* sk, int head_dim, int block_size,
                         Path path, const LaunchCtx& ctx);
// Records a kernel the current entry point enqueued (pa_last_launch).
void note_launch(const char* name);
// Address of the current device's copy of the library's fixed scratch array
// (PA_NOALLOC_SCRATCH_BYTES, 256-byte aligned), looked up once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
hipError_t launch_append(const AppendParams& p, int head_dim, int block_size, hipStream_t stream);
hipError_t launch_copy(const CopyParams& p, hipStream_t stream);
hipError_t launch_multi(const MultiParams& p, int head_dim, int block_size, const LaunchCtx& c);
// A decode step on the partitioned schedule (m.d's partitions, one new token
// per sequence in m): true where that schedule runs the shared-partition
// kernel, which then takes the append too (launch_shared_step: one launch and
// the combine; hipErrorInvalidValue where it does not apply).
bool shared_step_applies(const DecodeParams& p, Path path, const LaunchCtx& c);
hipError_t launch_shared_step(const MultiParams& m, int head_dim, int block_size, const LaunchCtx& c);
// Contiguous control: k_cache / v_cache hold one region of max_len tokens per
// (sequence, KV head); MFMA path, no split.
hipError_t launch_contiguous(const DecodeParams& p, int head_dim, const LaunchCtx& ctx);

}  // namespace pa
