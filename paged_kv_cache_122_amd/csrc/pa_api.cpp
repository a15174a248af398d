// Host side of libpa: argument validation, split-K planning, workspace
// management, debug-mode contract checks and kernel launches.  Implements the
// C ABI declared in include/pa.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_error;
thread_local std::string g_launch;  // kernels the last entry point enqueued on this thread
std::atomic<int> g_debug{0};

// Start of every entry point: no message, no launch yet.
void begin_call() {
  g_error.clear();
  g_launch.clear();
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

const char* dtype_name(int dt) {
  switch (dt) {
    case PA_BF16: return "bf16";
    case PA_F32: return "f32";
    case PA_I32: return "i32";
    case PA_I64: return "i64";
  }
  return "unknown";
}

int64_t numel(const pa_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Basic descriptor sanity: dtype, rank, non-negative shape, data present.
int check_desc(const pa_tensor* t, const char* name, int dtype, int ndim) {
  if (!t) return fail(PA_ERR_INVALID, "%s: descriptor is NULL", name);
  if (t->dtype != dtype)
    return fail(PA_ERR_INVALID, "%s: dtype %s, expected %s", name, dtype_name(t->dtype),
                dtype_name(dtype));
  if (t->ndim != ndim) return fail(PA_ERR_INVALID, "%s: %d dims, expected %d", name, t->ndim, ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0 || t->stride[i] < 0)
      return fail(PA_ERR_INVALID, "%s: negative shape or stride in dim %d", name, i);
  if (!t->data && numel(t) > 0) return fail(PA_ERR_INVALID, "%s: data pointer is NULL", name);
  return PA_OK;
}

bool is_contiguous(const pa_tensor* t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct CacheGeom {
  int64_t num_blocks, kv_heads, head_dim, block_size;
};

// Validate the two pools against the documented layout.
int check_caches(const pa_tensor* kc, const pa_tensor* vc, CacheGeom* g) {
  int rc;
  if ((rc = check_desc(kc, "k_cache", PA_BF16, 5)) != PA_OK) return rc;
  if ((rc = check_desc(vc, "v_cache", PA_BF16, 5)) != PA_OK) return rc;
  const int64_t nb = kc->shape[0], hkv = kc->shape[1], d8 = kc->shape[2], bs = kc->shape[3];
  if (kc->shape[4] != 8)
    return fail(PA_ERR_INVALID, "k_cache: last dim %lld, expected 8 (layout [NB,Hkv,D/8,B,8])",
                (long long)kc->shape[4]);
  const int64_t d = d8 * 8;
  if (vc->shape[0] != nb || vc->shape[1] != hkv || vc->shape[2] * 4 != bs || vc->shape[3] != d ||
      vc->shape[4] != 4)
    return fail(PA_ERR_INVALID,
                "v_cache: shape [%lld,%lld,%lld,%lld,%lld] does not match k_cache "
                "(expected [NB,Hkv,B/4,D,4] = [%lld,%lld,%lld,%lld,4])",
                (long long)vc->shape[0], (long long)vc->shape[1], (long long)vc->shape[2],
                (long long)vc->shape[3], (long long)vc->shape[4], (long long)nb, (long long)hkv,
                (long long)(bs / 4), (long long)d);
  if (!is_contiguous(kc) || !is_contiguous(vc))
    return fail(PA_ERR_INVALID, "k_cache/v_cache must be contiguous");
  if (d != 64 && d != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %lld (supported: 64, 128)", (long long)d);
  if (bs != 8 && bs != 16 && bs != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size %lld (supported: 8, 16, 32)", (long long)bs);
  if (hkv <= 0) return fail(PA_ERR_INVALID, "num_kv_heads must be positive");
  if (nb > 0 && (!aligned16(kc->data) || !aligned16(vc->data)))
    return fail(PA_ERR_INVALID, "k_cache/v_cache must be 16-byte aligned");
  g->num_blocks = nb;
  g->kv_heads = hkv;
  g->head_dim = d;
  g->block_size = bs;
  return PA_OK;
}

// Rows of a [T, H, D] bf16 tensor must be contiguous and 16-byte aligned.
int check_rows(const pa_tensor* t, const char* name) {
  if (t->stride[2] != 1 && t->shape[2] > 1)
    return fail(PA_ERR_INVALID, "%s: last dim must be contiguous", name);
  if (numel(t) > 0 && (!aligned16(t->data) || (t->stride[0] % 8) || (t->stride[1] % 8)))
    return fail(PA_ERR_INVALID, "%s: rows must be 16-byte aligned (strides multiple of 8)", name);
  return PA_OK;
}

template <typename T>
int copy_to_host(std::vector<T>* dst, const void* src, size_t n, hipStream_t stream) {
  dst->resize(n);
  if (n == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(dst->data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "debug copy to host");
  return PA_OK;
}

// ---------------------------------------------------------------------------
// library-owned decode workspace, one per device
// ---------------------------------------------------------------------------
// Partial results only: every split call writes each entry before the combine
// kernel reads it, so the buffer needs no initialisation and no call depends
// on what an earlier call left in it.
struct DeviceBuffer {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::unordered_map<int, DeviceBuffer> g_ws;

int grow(DeviceBuffer* b, size_t need, hipStream_t stream) {
  if (b->bytes >= need) return PA_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode needs %zu more workspace bytes but may not allocate during stream "
                "capture; use pa_decode_ex with a caller-owned workspace",
                need);
  if (b->ptr) {
    e = hipFree(b->ptr);  // synchronises the device: no queued kernel still uses it
    b->ptr = nullptr;
    b->bytes = 0;
    if (e != hipSuccess) return hip_fail(e, "hipFree(workspace)");
  }
  const size_t bytes = (need + need / 4 + 255) & ~size_t(255);
  e = hipMalloc(&b->ptr, bytes);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
  b->bytes = bytes;
  return PA_OK;
}

// Library-owned partial-result storage on the current device.
int owned_workspace(size_t need, hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceBuffer& w = g_ws[dev];
  const int rc = grow(&w, need, stream);
  if (rc != PA_OK) return rc;
  *out = w.ptr;
  return PA_OK;
}

struct DecodePlan {
  int64_t S, Hq, Hkv, D, B, W, NB;
  int part_tokens, max_parts;
  bool share_unsplit;   // automatic, unsplit, G <= 2: the shared-partition kernel where the grid fills the GPU
  bool stream;          // stream-K schedule (else partitioned)
  int workgroups_per_cu;
  pa::Path path;
  pa::WorkspaceLayout ws;
};

// The stream-K schedule keeps its tile prefix in LDS and indexes tiles with
// 32-bit integers: it takes the batch when both fit.
bool stream_fits(int64_t S, int64_t pairs, int64_t max_len) {
  const int64_t tiles = pairs * ((max_len + pa::kTileTokens - 1) / pa::kTileTokens);
  return S <= pa::kMaxStreamSeqs && tiles < (int64_t(1) << 30);
}

// Schedule of an automatic call, from shapes only (no device read, the same on
// every device so that pa_decode_workspace_bytes agrees with pa_decode_ex).
// Measured on MI355X with caches flushed:
//  * enough (sequence, head group) pairs to give every wave of a full GPU
//    (256 CUs x 8 waves) its own share -> one workgroup per pair, no split and
//    no combine launch (Llama-3-8B/70B-shaped batches);
//  * MHA (1-2 q heads per KV head) with that many pairs -> 1024-token
//    partitions, which keep the shared prefix blocks of neighbouring sequences
//    in flight together;
//  * tiny batches -> one workgroup per pair (the launch cost dominates);
//  * otherwise (few, long contexts) -> stream-K.
constexpr int64_t kFullGpuPairs = 512;
constexpr int64_t kNoSplitMaxLen = 8192;
// Few pairs: tables up to this many tokens stay unsplit; longer ones take
// partitions of kDefaultPartition tokens while their grid has at most
// kMaxPartitionGrid workgroups (most of it resident at once, so partitions a
// short context leaves empty cost little), and stream-K beyond.
constexpr int64_t kSmallNoSplitLen = 1024;
constexpr int64_t kMaxPartitionGrid = 2048;

struct Schedule {
  bool stream;
  int64_t part;  // partitioned: tokens per partition (-1 = one per sequence)
};

Schedule auto_schedule(int64_t S, int64_t pairs, int64_t group, int64_t max_len) {
  const int64_t tiles = (max_len + pa::kTileTokens - 1) / pa::kTileTokens;
  if (pairs >= kFullGpuPairs)
    return {false, group <= 2 ? 1024 : (max_len <= kNoSplitMaxLen ? -1 : 1024)};
  (void)tiles;
  if (max_len <= kSmallNoSplitLen) return {false, -1};
  const int64_t parts = (max_len + pa::kDefaultPartition - 1) / pa::kDefaultPartition;
  if (pairs * parts <= kMaxPartitionGrid) return {false, pa::kDefaultPartition};
  if (stream_fits(S, pairs, max_len)) return {true, 0};
  return {false, pa::kDefaultPartition};
}

// CUs of the current device (cached per device).
int device_cus(int* cus) {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    it = cache.emplace(dev, n > 0 ? n : 1).first;
  }
  *cus = it->second;
  return PA_OK;
}

int plan_decode(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                const pa_tensor* v_cache, const pa_tensor* block_tables,
                const pa_tensor* context_lens, int32_t block_size, const pa_decode_opts* opts,
                DecodePlan* pl) {
  int rc;
  CacheGeom g;
  if ((rc = check_caches(k_cache, v_cache, &g)) != PA_OK) return rc;
  if ((rc = check_desc(q, "q", PA_BF16, 3)) != PA_OK) return rc;
  if (!out) return fail(PA_ERR_INVALID, "out: descriptor is NULL");
  if (out->dtype != PA_BF16 && out->dtype != PA_F32)
    return fail(PA_ERR_INVALID, "out: dtype %s, expected bf16 or f32", dtype_name(out->dtype));
  if ((rc = check_desc(out, "out", out->dtype, 3)) != PA_OK) return rc;
  if ((rc = check_desc(block_tables, "block_tables", PA_I32, 2)) != PA_OK) return rc;
  if ((rc = check_desc(context_lens, "context_lens", PA_I32, 1)) != PA_OK) return rc;

  const int64_t S = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  if (D != g.head_dim)
    return fail(PA_ERR_INVALID, "q: head_dim %lld, caches have %lld", (long long)D, (long long)g.head_dim);
  if (out->shape[0] != S || out->shape[1] != Hq || out->shape[2] != D)
    return fail(PA_ERR_INVALID, "out: shape does not match q");
  if (block_size != g.block_size)
    return fail(PA_ERR_INVALID, "block_size %d does not match the caches' %lld", block_size,
                (long long)g.block_size);
  if (Hq <= 0 || Hq % g.kv_heads)
    return fail(PA_ERR_INVALID, "num_q_heads %lld is not a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)g.kv_heads);
  if (block_tables->shape[0] != S || context_lens->shape[0] != S)
    return fail(PA_ERR_INVALID, "block_tables/context_lens: first dim must be num_seqs %lld", (long long)S);
  const int64_t W = block_tables->shape[1];
  if (W < 1) return fail(PA_ERR_INVALID, "block_tables: width must be >= 1");
  if (block_tables->stride[1] != 1 || block_tables->stride[0] < W)
    return fail(PA_ERR_INVALID, "block_tables: rows must be contiguous with row stride >= width");
  if (context_lens->stride[0] != 1 && S > 1)
    return fail(PA_ERR_INVALID, "context_lens must be contiguous");
  if ((rc = check_rows(q, "q")) != PA_OK) return rc;
  if (out->stride[2] != 1 && D > 1) return fail(PA_ERR_INVALID, "out: last dim must be contiguous");
  if (S > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs %lld > 65535", (long long)S);

  const int64_t G = Hq / g.kv_heads;
  const int want = opts ? opts->path : 0;
  pa::Path path;
  if (want == 0)  // MFMA costs nothing on padding columns: faster than VALU also at G = 1, 2
    path = pa::Path::Mfma;
  else if (want == 1)
    path = pa::Path::Valu;
  else if (want == 2)
    path = pa::Path::Mfma;
  else
    return fail(PA_ERR_INVALID, "opts.path %d (expected 0, 1 or 2)", want);
  if (path == pa::Path::Valu && G > 2)
    return fail(PA_ERR_UNSUPPORTED, "the VALU path takes 1 or 2 query heads per KV head, not %lld",
                (long long)G);

  int64_t max_len = (opts && opts->max_context_len > 0) ? opts->max_context_len : W * g.block_size;
  if (opts && opts->max_context_len < 0) return fail(PA_ERR_INVALID, "opts.max_context_len < 0");
  if (opts && opts->max_context_len == 0 && opts->host_context_lens && S > 0) {
    // the longest context bounds the launch, not the table width (engines
    // often size tables for the model's maximum context)
    int64_t longest = 1;
    for (int64_t s = 0; s < S; ++s) longest = std::max<int64_t>(longest, opts->host_context_lens[s]);
    max_len = std::min(longest, max_len);
  }
  if (W * g.block_size > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "table width * block_size >= 2^31");
  const int pt_opt = opts ? opts->partition_tokens : 0;
  const int wpc = opts ? opts->workgroups_per_cu : 0;
  if (wpc < 0 || wpc > 64) return fail(PA_ERR_INVALID, "opts.workgroups_per_cu %d (0 .. 64)", wpc);
  if (opts && opts->reserved != 0) return fail(PA_ERR_INVALID, "opts.reserved must be 0");
  if (opts && (opts->kernel_start == nullptr) != (opts->kernel_stop == nullptr))
    return fail(PA_ERR_INVALID, "opts.kernel_start and opts.kernel_stop: both or neither");
  const int64_t head_groups = path == pa::Path::Mfma ? (G + 15) / 16 : 1;
  const int64_t pairs = S * g.kv_heads * head_groups;

  pl->S = S;
  pl->Hq = Hq;
  pl->Hkv = g.kv_heads;
  pl->D = D;
  pl->B = g.block_size;
  pl->W = W;
  pl->NB = g.num_blocks;
  pl->path = path;
  pl->workgroups_per_cu = wpc > 0 ? wpc : pa::kDefaultWorkgroupsPerCu;
  int64_t want_part;  // -2 stream-K, -1 one partition per sequence, > 0 partition tokens
  if (pt_opt == 0) {
    const Schedule sc = auto_schedule(S, S * g.kv_heads * ((G + 15) / 16), G, max_len);
    want_part = sc.stream ? -2 : sc.part;
  } else if (pt_opt == -1 || pt_opt == -2 || (pt_opt > 0 && pt_opt % 32 == 0)) {
    want_part = pt_opt;
  } else {
    return fail(PA_ERR_INVALID,
                "opts.partition_tokens %d (0, -1, -2 or a positive multiple of 32)", pt_opt);
  }
  if (want_part == -2) {
    if (!stream_fits(S, pairs, W * g.block_size))
      return fail(PA_ERR_UNSUPPORTED, "stream-K schedule: more than %d sequences or too many tiles",
                  pa::kMaxStreamSeqs);
    pl->stream = true;
    pl->part_tokens = 0;
    pl->max_parts = 1;
    pl->share_unsplit = false;
    pl->ws = pa::stream_workspace_layout(S, pairs, D);
    return PA_OK;
  }
  pl->stream = false;
  const int64_t part =
      want_part == -1 ? std::max<int64_t>(32, (max_len + 31) / 32 * 32) : want_part;
  if (part > (int64_t(1) << 30)) return fail(PA_ERR_UNSUPPORTED, "partition too large");
  const int64_t max_parts = std::max<int64_t>(1, (max_len + part - 1) / part);
  if (max_parts > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%lld partitions per sequence > 65535; raise partition_tokens",
                (long long)max_parts);

  pl->part_tokens = int(part);
  pl->max_parts = int(max_parts);
  // A split schedule with the automatic path takes the shared-partition
  // kernel for any grouping up to 16 where the grid fills the GPU: it reads a
  // partition that consecutive sequences share (a common prefix) once for all
  // of them.
  // Unsplit with one or two q heads per KV head: where the grid fills the GPU
  // the shared-partition kernel takes it (one partition spanning the table),
  // so that prefix blocks neighbouring sequences share (parallel samples of
  // a prompt) are read once; smaller grids take the MFMA decode.
  pl->share_unsplit = want == 0 && max_parts == 1 && G <= 2;
  pl->ws = pa::workspace_layout(S, Hq, D, max_parts);
  if (max_parts == 1) pl->ws.total = 0;
  return PA_OK;
}

int debug_check_decode(const DecodePlan& pl, const pa_tensor* block_tables,
                       const pa_tensor* context_lens, int64_t max_len, const int32_t* host_lens,
                       hipStream_t stream) {
  std::vector<int32_t> lens, bt;
  int rc;
  if ((rc = copy_to_host(&lens, context_lens->data, size_t(pl.S), stream)) != PA_OK) return rc;
  const size_t rows = size_t(pl.S), stride = size_t(block_tables->stride[0]);
  if ((rc = copy_to_host(&bt, block_tables->data, rows ? (rows - 1) * stride + size_t(pl.W) : 0, stream)) != PA_OK)
    return rc;
  for (int64_t s = 0; s < pl.S; ++s) {
    const int64_t L = lens[s];
    if (host_lens && host_lens[s] != L)
      return fail(PA_ERR_CONTRACT, "opts.host_context_lens[%lld] = %lld, but context_lens[%lld] = %lld",
                  (long long)s, (long long)host_lens[s], (long long)s, (long long)L);
    if (L < 0 || L > pl.W * pl.B)
      return fail(PA_ERR_CONTRACT, "context_lens[%lld] = %lld outside [0, width*block_size = %lld]",
                  (long long)s, (long long)L, (long long)(pl.W * pl.B));
    if (L > max_len)
      return fail(PA_ERR_CONTRACT, "context_lens[%lld] = %lld exceeds opts.max_context_len %lld",
                  (long long)s, (long long)L, (long long)max_len);
    const int64_t nblk = (L + pl.B - 1) / pl.B;
    for (int64_t i = 0; i < nblk; ++i) {
      const int64_t b = bt[size_t(s) * stride + size_t(i)];
      if (b < 0 || b >= pl.NB)
        return fail(PA_ERR_CONTRACT, "block_tables[%lld][%lld] = %lld outside [0, %lld)", (long long)s,
                    (long long)i, (long long)b, (long long)pl.NB);
    }
  }
  return PA_OK;
}

int decode_common(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                  const pa_tensor* v_cache, const pa_tensor* block_tables,
                  const pa_tensor* context_lens, float scale, int32_t block_size,
                  const pa_decode_opts* opts, bool owned_ws, void* workspace,
                  size_t workspace_bytes, bool debug, hipStream_t stream) {
  DecodePlan pl;
  int rc = plan_decode(out, q, k_cache, v_cache, block_tables, context_lens, block_size, opts, &pl);
  if (rc != PA_OK) return rc;
  if (pl.S == 0) return PA_OK;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "scale must be finite");
  const int64_t max_len = (opts && opts->max_context_len > 0) ? opts->max_context_len : pl.W * pl.B;
  if (debug && (rc = debug_check_decode(pl, block_tables, context_lens, max_len,
                                                   opts ? opts->host_context_lens : nullptr, stream)) != PA_OK)
    return rc;

  char* ws = nullptr;  // partial results of split contexts
  if (pl.ws.total > 0) {
    if (owned_ws) {
      void* w;
      if ((rc = owned_workspace(pl.ws.total, stream, &w)) != PA_OK) return rc;
      ws = static_cast<char*>(w);
    } else {
      if (!workspace || workspace_bytes < pl.ws.total)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                    pl.ws.total);
      if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
      ws = static_cast<char*>(workspace);
    }
  }

  pa::DecodeParams p{};
  p.out = out->data;
  p.out_s = out->stride[0];
  p.out_h = out->stride[1];
  p.out_f32 = out->dtype == PA_F32;
  p.q = static_cast<const uint16_t*>(q->data);
  p.q_s = q->stride[0];
  p.q_h = q->stride[1];
  p.k_cache = static_cast<const uint16_t*>(k_cache->data);
  p.v_cache = static_cast<const uint16_t*>(v_cache->data);
  p.block_tables = static_cast<const int32_t*>(block_tables->data);
  p.bt_s = block_tables->stride[0];
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.num_seqs = int(pl.S);
  p.num_q_heads = int(pl.Hq);
  p.num_kv_heads = int(pl.Hkv);
  p.group = int(pl.Hq / pl.Hkv);
  p.head_groups = pl.path == pa::Path::Mfma ? (p.group + 15) / 16 : 1;
  p.max_len = int(pl.W * pl.B);
  p.scale_log2 = float(double(scale) * 1.4426950408889634);
  p.part_tokens = pl.part_tokens;
  p.max_parts = pl.max_parts;
  p.share_unsplit = pl.share_unsplit;
  int cus = 0;
  if ((rc = device_cus(&cus)) != PA_OK) return rc;
  const pa::LaunchCtx ctx{stream, opts ? opts->kernel_start : nullptr,
                          opts ? opts->kernel_stop : nullptr, cus,
                          opts ? opts->host_context_lens : nullptr};
  hipError_t e;
  if (pl.stream) {
    pa::StreamParams sk{};
    sk.plan = reinterpret_cast<int*>(ws + pl.ws.plan_off);
    sk.ws_ml = reinterpret_cast<float*>(ws + pl.ws.ml_off);
    sk.ws_o = reinterpret_cast<float*>(ws + pl.ws.o_off);
    sk.cus = cus;
    sk.workgroups_per_cu = pl.workgroups_per_cu;
    e = pa::launch_decode(p, &sk, int(pl.D), int(pl.B), pl.path, ctx);
  } else {
    if (ws) {
      p.ws_ml = reinterpret_cast<float*>(ws + pl.ws.ml_off);
      p.ws_o = reinterpret_cast<float*>(ws + pl.ws.o_off);
    }
    e = pa::launch_decode(p, nullptr, int(pl.D), int(pl.B), pl.path, ctx);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return PA_OK;
}

}  // namespace

PA_EXPORT const char* pa_last_error(void) { return g_error.c_str(); }

PA_EXPORT const char* pa_last_launch(void) { return g_launch.c_str(); }

PA_EXPORT int pa_set_debug(int on) { return g_debug.exchange(on ? 1 : 0); }

PA_EXPORT size_t pa_decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads,
                                           int64_t num_kv_heads, int64_t head_dim,
                                           int64_t max_context_len, int32_t partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0)
    return 0;
  const int64_t group = num_q_heads / num_kv_heads;
  const int64_t pairs = num_seqs * num_kv_heads * ((group + 15) / 16);
  int64_t part = partition_tokens;
  if (part == 0) {
    const Schedule sc = auto_schedule(num_seqs, pairs, group, max_context_len);
    part = sc.stream ? -2 : sc.part;
  }
  if (part == -2)
    return stream_fits(num_seqs, pairs, max_context_len)
               ? pa::stream_workspace_layout(num_seqs, pairs, head_dim).total
               : 0;
  if (part <= 0) return 0;  // -1: one partition per sequence, nothing to combine
  const int64_t max_parts = std::max<int64_t>(1, (max_context_len + part - 1) / part);
  if (max_parts == 1) return 0;
  return pa::workspace_layout(num_seqs, num_q_heads, head_dim, max_parts).total;
}

PA_EXPORT int pa_decode_schedule(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                                 int64_t max_context_len, int32_t* partition_tokens) {
  g_error.clear();
  if (!partition_tokens) return fail(PA_ERR_INVALID, "partition_tokens is NULL");
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "bad sizes (S %lld, Hq %lld, Hkv %lld, max_context_len %lld)",
                (long long)num_seqs, (long long)num_q_heads, (long long)num_kv_heads,
                (long long)max_context_len);
  const int64_t group = num_q_heads / num_kv_heads;
  const Schedule sc =
      auto_schedule(num_seqs, num_seqs * num_kv_heads * ((group + 15) / 16), group, max_context_len);
  *partition_tokens = sc.stream ? -2 : int32_t(sc.part);
  return PA_OK;
}

PA_EXPORT int pa_decode(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                        const pa_tensor* v_cache, const pa_tensor* block_tables,
                        const pa_tensor* context_lens, float scale, int32_t block_size,
                        hipStream_t stream) {
  begin_call();
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       nullptr, true, nullptr, 0, g_debug.load() != 0, stream);
}

PA_EXPORT int pa_decode_ex(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                           const pa_tensor* v_cache, const pa_tensor* block_tables,
                           const pa_tensor* context_lens, float scale, int32_t block_size,
                           const pa_decode_opts* opts, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  begin_call();
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, opts,
                       false, workspace, workspace_bytes, g_debug.load() != 0, stream);
}

PA_EXPORT int pa_decode_noalloc(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                                const pa_tensor* v_cache, const pa_tensor* block_tables,
                                const pa_tensor* context_lens, float scale, int32_t block_size,
                                hipStream_t stream) {
  begin_call();
  // the size check comes before any device call: an oversized call launches nothing
  DecodePlan pl;
  int rc = plan_decode(out, q, k_cache, v_cache, block_tables, context_lens, block_size, nullptr, &pl);
  if (rc != PA_OK) return rc;
  if (pl.ws.total > PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_noalloc: this schedule needs %zu bytes of partial results, the library's "
                "fixed scratch holds %zu; use pa_decode_ex with a workspace",
                pl.ws.total, size_t(PA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (pl.S > 0 && pl.ws.total > 0) {
    const hipError_t e = pa::noalloc_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) return hip_fail(e, "looking up the scratch array of this device");
  }
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, nullptr,
                       false, ws, ws_bytes, g_debug.load() != 0, stream);
}

PA_EXPORT int pa_decode_contiguous(pa_tensor* out, const pa_tensor* q, const pa_tensor* k,
                                   const pa_tensor* v, const pa_tensor* context_lens, float scale,
                                   hipStream_t stream) {
  begin_call();
  int rc;
  if ((rc = check_desc(k, "k", PA_BF16, 5)) != PA_OK) return rc;
  if ((rc = check_desc(v, "v", PA_BF16, 5)) != PA_OK) return rc;
  if ((rc = check_desc(q, "q", PA_BF16, 3)) != PA_OK) return rc;
  if (!out) return fail(PA_ERR_INVALID, "out: descriptor is NULL");
  if (out->dtype != PA_BF16 && out->dtype != PA_F32)
    return fail(PA_ERR_INVALID, "out: dtype %s, expected bf16 or f32", dtype_name(out->dtype));
  if ((rc = check_desc(out, "out", out->dtype, 3)) != PA_OK) return rc;
  if ((rc = check_desc(context_lens, "context_lens", PA_I32, 1)) != PA_OK) return rc;
  const int64_t S = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  if (k->shape[2] * 8 != D || k->shape[3] != 16 || k->shape[4] != 8)
    return fail(PA_ERR_INVALID, "k: shape [S*Hkv, max_len/16, D/8, 16, 8] expected");
  if (S == 0 && k->shape[0] == 0) return PA_OK;
  if (S <= 0 || k->shape[0] % S)
    return fail(PA_ERR_INVALID, "k: first dim %lld is not num_seqs * num_kv_heads", (long long)k->shape[0]);
  const int64_t Hkv = k->shape[0] / S, Lmax = k->shape[1] * 16;
  const int64_t v_shape[5] = {k->shape[0], k->shape[1], 4, D, 4};
  for (int i = 0; i < 5; ++i)
    if (v->shape[i] != v_shape[i])
      return fail(PA_ERR_INVALID, "v: shape [S*Hkv, max_len/16, 4, D, 4] expected (matching k)");
  if (!is_contiguous(k) || !is_contiguous(v)) return fail(PA_ERR_INVALID, "k, v must be contiguous");
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %lld (64 or 128)", (long long)D);
  if (Lmax < 16 || Lmax * D * 2 >= (int64_t(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "max_len %lld (max_len * D * 2 must stay below 2^31)",
                (long long)Lmax);
  if (out->shape[0] != S || out->shape[1] != Hq || out->shape[2] != D)
    return fail(PA_ERR_INVALID, "out: shape does not match q");
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv)
    return fail(PA_ERR_INVALID, "num_q_heads %lld is not a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)Hkv);
  if (context_lens->shape[0] != S) return fail(PA_ERR_INVALID, "context_lens: %lld entries", (long long)S);
  if (context_lens->stride[0] != 1 && S > 1) return fail(PA_ERR_INVALID, "context_lens must be contiguous");
  if ((rc = check_rows(q, "q")) != PA_OK) return rc;
  if (out->stride[2] != 1 && D > 1) return fail(PA_ERR_INVALID, "out: last dim must be contiguous");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "scale must be finite");
  if (S > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs %lld > 65535", (long long)S);
  int cus = 0;
  if ((rc = device_cus(&cus)) != PA_OK) return rc;

  pa::DecodeParams p{};
  p.out = out->data;
  p.out_s = out->stride[0];
  p.out_h = out->stride[1];
  p.out_f32 = out->dtype == PA_F32;
  p.q = static_cast<const uint16_t*>(q->data);
  p.q_s = q->stride[0];
  p.q_h = q->stride[1];
  p.k_cache = static_cast<const uint16_t*>(k->data);
  p.v_cache = static_cast<const uint16_t*>(v->data);
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.num_seqs = int(S);
  p.num_q_heads = int(Hq);
  p.num_kv_heads = int(Hkv);
  p.group = int(Hq / Hkv);
  p.head_groups = (p.group + 15) / 16;
  p.max_len = int(Lmax);
  p.scale_log2 = float(double(scale) * 1.4426950408889634);
  p.part_tokens = int(Lmax);
  p.max_parts = 1;
  const pa::LaunchCtx ctx{stream, nullptr, nullptr, cus};
  const hipError_t e = pa::launch_contiguous(p, int(D), ctx);
  if (e != hipSuccess) return hip_fail(e, "contiguous decode launch");
  return PA_OK;
}

namespace {

// Kernel arguments of the multi-token kernel (shapes already validated);
// query_start may be NULL: one new token per sequence, row s.
// MFMA column sets and groups of a multi-token launch: columns are (new
// token, query head) pairs, at most 16 per set and two sets per workgroup.
void multi_columns(int64_t max_query_len, int64_t G, int* col_sets, int64_t* col_groups) {
  const int64_t cols = max_query_len * G;
  *col_sets = cols > 16 ? 2 : 1;
  *col_groups = (cols + 16 * *col_sets - 1) / (16 * *col_sets);
}

int multi_params(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_new, const pa_tensor* v_new,
                 const pa_tensor* slot_mapping, const pa_tensor* query_start, pa_tensor* k_cache,
                 pa_tensor* v_cache, const pa_tensor* block_tables, const pa_tensor* context_lens,
                 const CacheGeom& g, float scale, int32_t max_query_len, pa::MultiParams* mp) {
  const int64_t T = q->shape[0], Hq = q->shape[1], S = context_lens->shape[0];
  const int64_t G = Hq / g.kv_heads, W = block_tables->shape[1];
  int col_sets = 1;
  int64_t col_groups = 1;
  multi_columns(max_query_len, G, &col_sets, &col_groups);
  if (g.kv_heads * col_groups > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  pa::MultiParams m{};
  pa::DecodeParams& p = m.d;
  p.out = out->data;
  p.out_s = out->stride[0];
  p.out_h = out->stride[1];
  p.out_f32 = out->dtype == PA_F32;
  p.q = static_cast<const uint16_t*>(q->data);
  p.q_s = q->stride[0];
  p.q_h = q->stride[1];
  p.k_cache = static_cast<const uint16_t*>(k_cache->data);
  p.v_cache = static_cast<const uint16_t*>(v_cache->data);
  p.block_tables = static_cast<const int32_t*>(block_tables->data);
  p.bt_s = block_tables->stride[0];
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.num_seqs = int(S);
  p.num_q_heads = int(Hq);
  p.num_kv_heads = int(g.kv_heads);
  p.group = int(G);
  p.head_groups = 1;
  p.max_len = int(W * g.block_size);
  p.scale_log2 = float(double(scale) * 1.4426950408889634);
  p.part_tokens = p.max_len;
  p.max_parts = 1;
  m.k_new = static_cast<const uint16_t*>(k_new->data);
  m.v_new = static_cast<const uint16_t*>(v_new->data);
  m.kn_t = k_new->stride[0];
  m.kn_h = k_new->stride[1];
  m.vn_t = v_new->stride[0];
  m.vn_h = v_new->stride[1];
  m.slots = static_cast<const int64_t*>(slot_mapping->data);
  m.k_store = static_cast<uint16_t*>(k_cache->data);
  m.v_store = static_cast<uint16_t*>(v_cache->data);
  m.query_start = query_start ? static_cast<const int32_t*>(query_start->data) : nullptr;
  m.num_rows = int(T);
  m.max_query_len = max_query_len;
  m.col_sets = col_sets;
  m.col_groups = int(col_groups);
  m.num_slots = g.num_blocks * g.block_size;
  *mp = m;
  return PA_OK;
}

// Device-side contracts of pa_decode_multi, checked on the host.
int debug_check_multi(const pa_tensor* slot_mapping, const pa_tensor* query_start,
                      const pa_tensor* block_tables, const pa_tensor* context_lens, int64_t S,
                      int64_t T, int64_t W, int64_t B, int64_t NB, int64_t max_query_len,
                      hipStream_t stream) {
  std::vector<int32_t> lens, qs, bt;
  std::vector<int64_t> slots;
  int rc;
  if ((rc = copy_to_host(&lens, context_lens->data, size_t(S), stream)) != PA_OK) return rc;
  if ((rc = copy_to_host(&qs, query_start->data, size_t(S + 1), stream)) != PA_OK) return rc;
  if ((rc = copy_to_host(&slots, slot_mapping->data, size_t(T), stream)) != PA_OK) return rc;
  const size_t stride = size_t(block_tables->stride[0]);
  if ((rc = copy_to_host(&bt, block_tables->data, S ? size_t(S - 1) * stride + size_t(W) : 0, stream)) != PA_OK)
    return rc;
  if (qs[0] < 0 || qs[size_t(S)] > T)
    return fail(PA_ERR_CONTRACT, "query_start spans [%d, %d), outside [0, %lld)", qs[0], qs[size_t(S)],
                (long long)T);
  std::unordered_set<int64_t> written;
  for (int64_t s = 0; s < S; ++s) {
    const int64_t L = lens[size_t(s)], n = int64_t(qs[size_t(s + 1)]) - qs[size_t(s)];
    if (L < 0 || L > W * B)
      return fail(PA_ERR_CONTRACT, "context_lens[%lld] = %lld outside [0, width*block_size = %lld]",
                  (long long)s, (long long)L, (long long)(W * B));
    if (n < 0) return fail(PA_ERR_CONTRACT, "query_start decreases at %lld", (long long)s);
    if (n > L || n > max_query_len)
      return fail(PA_ERR_CONTRACT, "sequence %lld brings %lld tokens (context %lld, max_query_len %lld)",
                  (long long)s, (long long)n, (long long)L, (long long)max_query_len);
    for (int64_t i = 0; i < (L + B - 1) / B; ++i) {
      const int64_t b = bt[size_t(s) * stride + size_t(i)];
      if (b < 0 || b >= NB)
        return fail(PA_ERR_CONTRACT, "block_tables[%lld][%lld] = %lld outside [0, %lld)", (long long)s,
                    (long long)i, (long long)b, (long long)NB);
    }
    for (int64_t i = 0; i < n; ++i) {
      const int64_t pos = L - n + i;
      const int64_t sl = slots[size_t(qs[size_t(s)] + i)];
      if (sl < 0) continue;
      const int64_t want = int64_t(bt[size_t(s) * stride + size_t(pos / B)]) * B + pos % B;
      if (sl != want)
        return fail(PA_ERR_CONTRACT, "slot_mapping[%lld] = %lld, but position %lld of sequence %lld is slot %lld",
                    (long long)(qs[size_t(s)] + i), (long long)sl, (long long)pos, (long long)s, (long long)want);
      if (!written.insert(sl).second)
        return fail(PA_ERR_CONTRACT, "slot %lld is written twice", (long long)sl);
    }
  }
  // no cached token read by this call lies in a slot it writes
  for (int64_t s = 0; s < S && !written.empty(); ++s) {
    const int64_t L = lens[size_t(s)], n = int64_t(qs[size_t(s + 1)]) - qs[size_t(s)];
    for (int64_t pos = 0; pos < L - n; ++pos) {
      const int64_t sl = int64_t(bt[size_t(s) * stride + size_t(pos / B)]) * B + pos % B;
      if (written.count(sl))
        return fail(PA_ERR_CONTRACT, "sequence %lld reads slot %lld, which this call writes", (long long)s,
                    (long long)sl);
    }
  }
  return PA_OK;
}

}  // namespace

namespace {

// Partitions of the multi-token kernel sized on the host's lengths, so that
// about kFullGpuPairs workgroups share the tokens evenly: their size, count
// and, within the limits of the kernel-argument list, the (sequence,
// partition) items that hold tokens, longest contexts first.  Returns false
// where every context fits one partition (then the unsplit kernel is the
// better launch).  A grid over every sequence's table span would leave most
// workgroups of an uneven batch with nothing to do but load their length and
// leave.  Each sequence's count is the kernel's: its cached tokens (all but
// its `new_tokens` new ones) in partitions of `part`, at least one; with
// new_tokens 0 (counts unknown to the host) an upper bound, whose surplus
// items find no tokens and leave.
bool host_length_split(int64_t S, int64_t Hkv, int64_t span, const int32_t* host_lens, int64_t new_tokens,
                       pa::MultiParams* m) {
  auto len = [&](int64_t i) { return std::min<int64_t>(std::max<int64_t>(host_lens[i], 0), span); };
  int64_t tokens = 0, longest = 0;
  for (int64_t s = 0; s < S; ++s) {
    tokens += len(s);
    longest = std::max(longest, len(s));
  }
  const int64_t row_wgs = Hkv * m->col_groups;
  int64_t part = std::max<int64_t>(512, ((tokens * row_wgs + kFullGpuPairs - 1) / kFullGpuPairs + 255) / 256 * 256);
  while ((span + part - 1) / part > 65535) part *= 2;
  if (longest - new_tokens <= part) return false;
  const int64_t parts = (span + part - 1) / part;
  m->d.part_tokens = int(part);
  m->d.max_parts = int(parts);
  if (S <= pa::kMaxItemSeqs && parts <= 256) {
    std::vector<int> idx(static_cast<size_t>(S));
    for (int64_t i = 0; i < S; ++i) idx[size_t(i)] = int(i);
    std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return len(x) > len(y); });
    int items = 0;
    for (const int sq : idx) {
      const int64_t cached = std::max<int64_t>(len(sq) - new_tokens, 0);
      const int64_t np = std::min<int64_t>(std::max<int64_t>((cached + part - 1) / part, 1), parts);
      if (items + np > pa::kMaxOrder) {
        items = -1;
        break;
      }
      for (int64_t j = 0; j < np; ++j) m->d.order[items++] = uint16_t((sq << 8) | int(j));
    }
    if (items > 0) {
      m->d.has_order = 2;
      m->num_items = items;
    }
  }
  return true;
}

// The automatic split of a multi-token launch: when its grid would fill less
// than half the GPU, partitions (multiples of 256 tokens, at least 512) so
// that the workgroups cover the cached context about twice; 0 = no split.
int64_t multi_auto_part(int64_t pairs, int64_t max_len) {
  if (pairs >= kFullGpuPairs) return 0;
  const int64_t want = (kFullGpuPairs + pairs - 1) / pairs;
  int64_t part = std::max<int64_t>(512, ((max_len + want - 1) / want + 255) / 256 * 256);
  while ((max_len + part - 1) / part > 65535) part *= 2;
  return part < max_len ? part : 0;
}

// The multi-token launch as planned (with the caller's timing events).
int launch_multi_plan(const pa::MultiParams& m, const pa_decode_opts* opts, int64_t D, int64_t B,
                      const int32_t* host_lens, hipStream_t stream) {
  int cus = 0;
  int rc;
  if ((rc = device_cus(&cus)) != PA_OK) return rc;
  const pa::LaunchCtx ctx{stream, opts ? opts->kernel_start : nullptr, opts ? opts->kernel_stop : nullptr, cus,
                          host_lens};
  const hipError_t e = pa::launch_multi(m, int(D), int(B), ctx);
  if (e != hipSuccess) return hip_fail(e, "multi-token decode launch");
  return PA_OK;
}

// pa_decode_multi and pa_decode_multi_ex: `owned` takes the library
// workspace, else the caller's.
int multi_common(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_new, const pa_tensor* v_new,
                 const pa_tensor* slot_mapping, const pa_tensor* query_start, pa_tensor* k_cache,
                 pa_tensor* v_cache, const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                 int32_t block_size, int32_t max_query_len, const pa_decode_opts* opts, bool owned,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc;
  CacheGeom g;
  if ((rc = check_caches(k_cache, v_cache, &g)) != PA_OK) return rc;
  if ((rc = check_desc(q, "q", PA_BF16, 3)) != PA_OK) return rc;
  if ((rc = check_desc(k_new, "k_new", PA_BF16, 3)) != PA_OK) return rc;
  if ((rc = check_desc(v_new, "v_new", PA_BF16, 3)) != PA_OK) return rc;
  if (!out) return fail(PA_ERR_INVALID, "out: descriptor is NULL");
  if (out->dtype != PA_BF16 && out->dtype != PA_F32)
    return fail(PA_ERR_INVALID, "out: dtype %s, expected bf16 or f32", dtype_name(out->dtype));
  if ((rc = check_desc(out, "out", out->dtype, 3)) != PA_OK) return rc;
  if ((rc = check_desc(slot_mapping, "slot_mapping", PA_I64, 1)) != PA_OK) return rc;
  if ((rc = check_desc(query_start, "query_start", PA_I32, 1)) != PA_OK) return rc;
  if ((rc = check_desc(block_tables, "block_tables", PA_I32, 2)) != PA_OK) return rc;
  if ((rc = check_desc(context_lens, "context_lens", PA_I32, 1)) != PA_OK) return rc;

  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2], S = context_lens->shape[0];
  if (D != g.head_dim)
    return fail(PA_ERR_INVALID, "q: head_dim %lld, caches have %lld", (long long)D, (long long)g.head_dim);
  if (out->shape[0] != T || out->shape[1] != Hq || out->shape[2] != D)
    return fail(PA_ERR_INVALID, "out: shape does not match q");
  for (const pa_tensor* t : {k_new, v_new})
    if (t->shape[0] != T || t->shape[1] != g.kv_heads || t->shape[2] != D)
      return fail(PA_ERR_INVALID, "k_new/v_new: shape [%lld, %lld, %lld] expected", (long long)T,
                  (long long)g.kv_heads, (long long)D);
  if (slot_mapping->shape[0] != T || (slot_mapping->stride[0] != 1 && T > 1))
    return fail(PA_ERR_INVALID, "slot_mapping: %lld contiguous entries expected", (long long)T);
  if (query_start->shape[0] != S + 1 || (query_start->stride[0] != 1 && S > 0))
    return fail(PA_ERR_INVALID, "query_start: %lld contiguous entries expected", (long long)(S + 1));
  if (block_size != g.block_size)
    return fail(PA_ERR_INVALID, "block_size %d does not match the caches' %lld", block_size,
                (long long)g.block_size);
  if (Hq <= 0 || Hq % g.kv_heads)
    return fail(PA_ERR_INVALID, "num_q_heads %lld is not a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)g.kv_heads);
  if (block_tables->shape[0] != S)
    return fail(PA_ERR_INVALID, "block_tables: first dim must be num_seqs %lld", (long long)S);
  const int64_t W = block_tables->shape[1];
  if (W < 1) return fail(PA_ERR_INVALID, "block_tables: width must be >= 1");
  if (block_tables->stride[1] != 1 || block_tables->stride[0] < W)
    return fail(PA_ERR_INVALID, "block_tables: rows must be contiguous with row stride >= width");
  if (context_lens->stride[0] != 1 && S > 1) return fail(PA_ERR_INVALID, "context_lens must be contiguous");
  if ((rc = check_rows(q, "q")) != PA_OK) return rc;
  if ((rc = check_rows(k_new, "k_new")) != PA_OK) return rc;
  if ((rc = check_rows(v_new, "v_new")) != PA_OK) return rc;
  if (out->stride[2] != 1 && D > 1) return fail(PA_ERR_INVALID, "out: last dim must be contiguous");
  const int64_t G = Hq / g.kv_heads;
  if (max_query_len < 0 || int64_t(max_query_len) * G > (int64_t(1) << 24))
    return fail(PA_ERR_INVALID, "max_query_len %d (0 .. 2^24 / query heads per KV head)", max_query_len);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "scale must be finite");
  if (S > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs %lld > 65535", (long long)S);
  if (T > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "too many rows");
  if (W * g.block_size > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "table width * block_size >= 2^31");
  if (opts) {
    if (opts->reserved != 0) return fail(PA_ERR_INVALID, "opts.reserved must be 0");
    if (opts->path == 1) return fail(PA_ERR_UNSUPPORTED, "the multi-token path runs on MFMA only (opts.path 0 or 2)");
    if (opts->path != 0 && opts->path != 2) return fail(PA_ERR_INVALID, "opts.path %d (expected 0 or 2)", opts->path);
    if (opts->workgroups_per_cu != 0) return fail(PA_ERR_INVALID, "opts.workgroups_per_cu must be 0 here");
    if (opts->partition_tokens == -2) return fail(PA_ERR_UNSUPPORTED, "no stream-K schedule for several new tokens");
    if (opts->partition_tokens < -2 || (opts->partition_tokens > 0 && opts->partition_tokens % 32))
      return fail(PA_ERR_INVALID, "opts.partition_tokens %d (0, -1 or a positive multiple of 32)",
                  opts->partition_tokens);
    if (opts->max_context_len < 0) return fail(PA_ERR_INVALID, "opts.max_context_len < 0");
    if ((opts->kernel_start == nullptr) != (opts->kernel_stop == nullptr))
      return fail(PA_ERR_INVALID, "opts.kernel_start and opts.kernel_stop: both or neither");
  }
  const int32_t* host_lens = opts ? opts->host_context_lens : nullptr;
  if (S == 0 || T == 0 || max_query_len == 0) return PA_OK;
  if (g_debug.load()) {
    if ((rc = debug_check_multi(slot_mapping, query_start, block_tables, context_lens, S, T, W, g.block_size,
                                g.num_blocks, max_query_len, stream)) != PA_OK)
      return rc;
    if (host_lens) {
      std::vector<int32_t> lens;
      if ((rc = copy_to_host(&lens, context_lens->data, size_t(S), stream)) != PA_OK) return rc;
      for (int64_t s = 0; s < S; ++s)
        if (host_lens[s] != lens[size_t(s)])
          return fail(PA_ERR_CONTRACT, "opts.host_context_lens[%lld] = %lld, but context_lens[%lld] = %lld",
                      (long long)s, (long long)host_lens[s], (long long)s, (long long)lens[size_t(s)]);
    }
  }

  pa::MultiParams m;
  if ((rc = multi_params(out, q, k_new, v_new, slot_mapping, query_start, k_cache, v_cache, block_tables,
                         context_lens, g, scale, max_query_len, &m)) != PA_OK)
    return rc;
  // the bound on the cached context that sizes a split: opts, else the
  // longest host length, else the table width
  int64_t max_len = W * g.block_size;
  if (opts && opts->max_context_len > 0) {
    max_len = opts->max_context_len;
  } else if (host_lens) {
    int64_t longest = 1;
    for (int64_t s = 0; s < S; ++s) longest = std::max<int64_t>(longest, host_lens[s]);
    max_len = std::min(longest, max_len);
  }
  const int64_t pairs = S * g.kv_heads * m.col_groups;
  const int32_t want = opts ? opts->partition_tokens : 0;
  if (host_lens && want == 0 && pairs < kFullGpuPairs) {
    // automatic split with the host's lengths: partitions sized on them and
    // only those holding tokens launched (as pa_append_decode), or no split
    // where every context fits one; the shape-only split below where the
    // caller's workspace is too small for that plan
    pa::MultiParams hm = m;
    if (!host_length_split(S, g.kv_heads, W * g.block_size, host_lens, 0, &hm))
      return launch_multi_plan(m, opts, D, g.block_size, host_lens, stream);
    const pa::WorkspaceLayout wl = pa::workspace_layout(T, Hq, D, hm.d.max_parts);
    void* ws = nullptr;
    if (owned) {
      if ((rc = owned_workspace(wl.total, stream, &ws)) != PA_OK) return rc;
    } else if (workspace && workspace_bytes >= wl.total && !(reinterpret_cast<uintptr_t>(workspace) & 255u)) {
      ws = workspace;
    }
    if (ws) {
      hm.d.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.ml_off);
      hm.d.ws_o = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.o_off);
      return launch_multi_plan(hm, opts, D, g.block_size, host_lens, stream);
    }
  }
  int64_t part = want == 0 ? multi_auto_part(pairs, max_len) : (want > 0 && want < max_len ? want : 0);
  if (part > 0) {
    const int64_t parts = (max_len + part - 1) / part;
    if (parts > 65535) return fail(PA_ERR_INVALID, "opts.partition_tokens %lld: more than 65535 partitions", (long long)part);
    const pa::WorkspaceLayout wl = pa::workspace_layout(T, Hq, D, parts);
    void* ws = nullptr;
    if (owned) {
      if ((rc = owned_workspace(wl.total, stream, &ws)) != PA_OK) return rc;
    } else {
      if (!workspace || workspace_bytes < wl.total)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, wl.total);
      if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
      ws = workspace;
    }
    m.d.part_tokens = int(part);
    m.d.max_parts = int(parts);
    m.d.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.ml_off);
    m.d.ws_o = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.o_off);
  }
  return launch_multi_plan(m, opts, D, g.block_size, host_lens, stream);
}

}  // namespace

PA_EXPORT int pa_decode_multi(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_new,
                              const pa_tensor* v_new, const pa_tensor* slot_mapping,
                              const pa_tensor* query_start, pa_tensor* k_cache, pa_tensor* v_cache,
                              const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                              int32_t block_size, int32_t max_query_len, hipStream_t stream) {
  begin_call();
  return multi_common(out, q, k_new, v_new, slot_mapping, query_start, k_cache, v_cache, block_tables,
                      context_lens, scale, block_size, max_query_len, nullptr, true, nullptr, 0, stream);
}

PA_EXPORT int pa_decode_multi_ex(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_new,
                                 const pa_tensor* v_new, const pa_tensor* slot_mapping,
                                 const pa_tensor* query_start, pa_tensor* k_cache, pa_tensor* v_cache,
                                 const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                                 int32_t block_size, int32_t max_query_len, const pa_decode_opts* opts,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  begin_call();
  return multi_common(out, q, k_new, v_new, slot_mapping, query_start, k_cache, v_cache, block_tables,
                      context_lens, scale, block_size, max_query_len, opts, false, workspace, workspace_bytes,
                      stream);
}

PA_EXPORT size_t pa_decode_multi_workspace_bytes(int64_t num_rows, int64_t num_seqs, int64_t num_q_heads,
                                                 int64_t num_kv_heads, int64_t head_dim, int32_t max_query_len,
                                                 int64_t max_context_len, int32_t partition_tokens) {
  if (num_rows <= 0 || num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads ||
      max_query_len <= 0 || max_context_len <= 0 || head_dim <= 0)
    return 0;
  int col_sets = 1;
  int64_t col_groups = 1;
  multi_columns(max_query_len, num_q_heads / num_kv_heads, &col_sets, &col_groups);
  const int64_t pairs = num_seqs * num_kv_heads * col_groups;
  const int64_t part = partition_tokens == 0 ? multi_auto_part(pairs, max_context_len)
                                             : (partition_tokens > 0 && partition_tokens < max_context_len
                                                    ? partition_tokens : 0);
  if (part <= 0) return 0;
  return pa::workspace_layout(num_rows, num_q_heads, head_dim, (max_context_len + part - 1) / part).total;
}

namespace {

// pa_cache_append's work; `debug` checks the slot contract first.
int cache_append_impl(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping, pa_tensor* k_cache,
                      pa_tensor* v_cache, bool debug, hipStream_t stream) {
  int rc;
  CacheGeom g;
  if ((rc = check_caches(k_cache, v_cache, &g)) != PA_OK) return rc;
  if ((rc = check_desc(k, "k", PA_BF16, 3)) != PA_OK) return rc;
  if ((rc = check_desc(v, "v", PA_BF16, 3)) != PA_OK) return rc;
  if ((rc = check_desc(slot_mapping, "slot_mapping", PA_I64, 1)) != PA_OK) return rc;
  const int64_t T = k->shape[0];
  if (k->shape[1] != g.kv_heads || k->shape[2] != g.head_dim)
    return fail(PA_ERR_INVALID, "k: shape [T, %lld, %lld] expected", (long long)g.kv_heads,
                (long long)g.head_dim);
  if (v->shape[0] != T || v->shape[1] != g.kv_heads || v->shape[2] != g.head_dim)
    return fail(PA_ERR_INVALID, "v: shape must equal k's");
  if (slot_mapping->shape[0] != T)
    return fail(PA_ERR_INVALID, "slot_mapping: %lld entries for %lld tokens",
                (long long)slot_mapping->shape[0], (long long)T);
  if (slot_mapping->stride[0] != 1 && T > 1) return fail(PA_ERR_INVALID, "slot_mapping must be contiguous");
  if ((rc = check_rows(k, "k")) != PA_OK) return rc;
  if ((rc = check_rows(v, "v")) != PA_OK) return rc;
  if (T == 0) return PA_OK;
  if (T > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "too many tokens");

  if (debug) {
    std::vector<int64_t> slots;
    if ((rc = copy_to_host(&slots, slot_mapping->data, size_t(T), stream)) != PA_OK) return rc;
    std::unordered_set<int64_t> seen;
    const int64_t nslots = g.num_blocks * g.block_size;
    for (int64_t i = 0; i < T; ++i) {
      const int64_t sl = slots[size_t(i)];
      if (sl < 0) continue;
      if (sl >= nslots)
        return fail(PA_ERR_CONTRACT, "slot_mapping[%lld] = %lld outside [0, %lld)", (long long)i,
                    (long long)sl, (long long)nslots);
      if (!seen.insert(sl).second)
        return fail(PA_ERR_CONTRACT, "slot_mapping[%lld] = %lld repeats an earlier slot", (long long)i,
                    (long long)sl);
    }
  }

  pa::AppendParams p{};
  p.k = static_cast<const uint16_t*>(k->data);
  p.v = static_cast<const uint16_t*>(v->data);
  p.k_t = k->stride[0];
  p.k_h = k->stride[1];
  p.v_t = v->stride[0];
  p.v_h = v->stride[1];
  p.slots = static_cast<const int64_t*>(slot_mapping->data);
  p.k_cache = static_cast<uint16_t*>(k_cache->data);
  p.v_cache = static_cast<uint16_t*>(v_cache->data);
  p.num_tokens = int(T);
  p.num_kv_heads = int(g.kv_heads);
  const hipError_t e = pa::launch_append(p, int(g.head_dim), int(g.block_size), stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return PA_OK;
}

}  // namespace

namespace {

// pa_append_decode's slot contract (debug mode): the slot of a sequence with
// tokens is its table's slot of position L - 1; an empty sequence has none.
int debug_check_append_slots(const DecodePlan& pl, const pa_tensor* slot_mapping, const pa_tensor* block_tables,
                             const pa_tensor* context_lens, hipStream_t stream) {
  std::vector<int32_t> lens, bt;
  std::vector<int64_t> slots;
  const size_t stride = size_t(block_tables->stride[0]);
  int rc;
  if ((rc = copy_to_host(&lens, context_lens->data, size_t(pl.S), stream)) != PA_OK) return rc;
  if ((rc = copy_to_host(&slots, slot_mapping->data, size_t(pl.S), stream)) != PA_OK) return rc;
  if ((rc = copy_to_host(&bt, block_tables->data, size_t(pl.S - 1) * stride + size_t(pl.W), stream)) != PA_OK)
    return rc;
  for (int64_t s = 0; s < pl.S; ++s) {
    const int64_t L = lens[size_t(s)];
    if (L == 0) {
      if (slots[size_t(s)] >= 0)
        return fail(PA_ERR_CONTRACT, "sequence %lld has no token (context length 0) but slot %lld",
                    (long long)s, (long long)slots[size_t(s)]);
      continue;
    }
    const int64_t want = int64_t(bt[size_t(s) * stride + size_t((L - 1) / pl.B)]) * pl.B + (L - 1) % pl.B;
    if (slots[size_t(s)] != want)
      return fail(PA_ERR_CONTRACT, "slot_mapping[%lld] = %lld, but position %lld of sequence %lld is slot %lld",
                  (long long)s, (long long)slots[size_t(s)], (long long)(L - 1), (long long)s, (long long)want);
  }
  return PA_OK;
}

// pa_append_decode's read contract (debug mode): no sequence reads a slot
// that this call writes for another sequence (a block receiving a new token
// is private to its sequence, as copy-on-write leaves it).
int debug_check_append_reads(const DecodePlan& pl, const pa_tensor* slot_mapping, const pa_tensor* block_tables,
                             const pa_tensor* context_lens, hipStream_t stream) {
  std::vector<int32_t> lens, bt;
  std::vector<int64_t> slots;
  const size_t stride = size_t(block_tables->stride[0]);
  int rc;
  if ((rc = copy_to_host(&lens, context_lens->data, size_t(pl.S), stream)) != PA_OK) return rc;
  if ((rc = copy_to_host(&slots, slot_mapping->data, size_t(pl.S), stream)) != PA_OK) return rc;
  if ((rc = copy_to_host(&bt, block_tables->data, size_t(pl.S - 1) * stride + size_t(pl.W), stream)) != PA_OK)
    return rc;
  std::unordered_map<int64_t, int64_t> writer;  // slot -> the sequence whose new token it receives
  for (int64_t s = 0; s < pl.S; ++s)
    if (slots[size_t(s)] >= 0) writer[slots[size_t(s)]] = s;
  for (int64_t c = 0; c < pl.S && !writer.empty(); ++c) {
    const int64_t L = std::min<int64_t>(std::max<int32_t>(lens[size_t(c)], 0), pl.W * pl.B);
    for (int64_t pos = 0; pos < L; ++pos) {
      const int64_t sl = int64_t(bt[size_t(c) * stride + size_t(pos / pl.B)]) * pl.B + pos % pl.B;
      const auto it = writer.find(sl);
      if (it != writer.end() && it->second != c)
        return fail(PA_ERR_CONTRACT,
                    "sequence %lld reads slot %lld (position %lld), which receives the new token of sequence %lld",
                    (long long)c, (long long)sl, (long long)pos, (long long)it->second);
    }
  }
  return PA_OK;
}

// One launch of the multi-token kernel for the step (one new token per
// sequence): it stores the new token and attends, taking its K/V from k and
// v; split (m->d.max_parts > 1, pieces in the workspace) a combine follows.
int launch_fused_step(const DecodePlan& pl, pa::MultiParams* m, const pa_decode_opts* opts, void* workspace,
                      hipStream_t stream) {
  int rc;
  if (m->d.max_parts > 1) {
    const pa::WorkspaceLayout wl = pa::workspace_layout(pl.S, pl.Hq, pl.D, m->d.max_parts);
    m->d.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
    m->d.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
  }
  int cus = 0;
  if ((rc = device_cus(&cus)) != PA_OK) return rc;
  const pa::LaunchCtx ctx{stream, opts ? opts->kernel_start : nullptr, opts ? opts->kernel_stop : nullptr, cus,
                          opts ? opts->host_context_lens : nullptr};
  const hipError_t e = pa::launch_multi(*m, int(pl.D), int(pl.B), ctx);
  if (e != hipSuccess) return hip_fail(e, "fused append + decode launch");
  return PA_OK;
}

}  // namespace

PA_EXPORT int pa_append_decode(pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                               const pa_tensor* slot_mapping, pa_tensor* k_cache, pa_tensor* v_cache,
                               const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                               int32_t block_size, const pa_decode_opts* opts, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  begin_call();
  int rc;
  DecodePlan pl;
  if ((rc = plan_decode(out, q, k_cache, v_cache, block_tables, context_lens, block_size, opts, &pl)) != PA_OK)
    return rc;
  if ((rc = check_desc(k, "k", PA_BF16, 3)) != PA_OK) return rc;
  if ((rc = check_desc(v, "v", PA_BF16, 3)) != PA_OK) return rc;
  if ((rc = check_desc(slot_mapping, "slot_mapping", PA_I64, 1)) != PA_OK) return rc;
  for (const pa_tensor* t : {k, v})
    if (t->shape[0] != pl.S || t->shape[1] != pl.Hkv || t->shape[2] != pl.D)
      return fail(PA_ERR_INVALID, "k/v: shape [%lld, %lld, %lld] expected (one new token per sequence)",
                  (long long)pl.S, (long long)pl.Hkv, (long long)pl.D);
  if (slot_mapping->shape[0] != pl.S || (slot_mapping->stride[0] != 1 && pl.S > 1))
    return fail(PA_ERR_INVALID, "slot_mapping: %lld contiguous entries expected", (long long)pl.S);
  if ((rc = check_rows(k, "k")) != PA_OK) return rc;
  if ((rc = check_rows(v, "v")) != PA_OK) return rc;
  if (pl.S == 0) return PA_OK;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "scale must be finite");
  // everything the decode will check, checked before the append launches
  if (pl.ws.total > 0) {
    if (!workspace || workspace_bytes < pl.ws.total)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, pl.ws.total);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int32_t* host_lens = opts ? opts->host_context_lens : nullptr;
  if (g_debug.load()) {
    const int64_t max_len = (opts && opts->max_context_len > 0) ? opts->max_context_len : pl.W * pl.B;
    if ((rc = debug_check_decode(pl, block_tables, context_lens, max_len, host_lens, stream)) != PA_OK) return rc;
    if ((rc = debug_check_append_slots(pl, slot_mapping, block_tables, context_lens, stream)) != PA_OK) return rc;
    if ((rc = debug_check_append_reads(pl, slot_mapping, block_tables, context_lens, stream)) != PA_OK) return rc;
  }

  // Route: the multi-token kernel in one launch where the schedule is unsplit
  // on the MFMA path (unless the shared-partition kernel takes the unsplit
  // grid, below); with host lengths, also where the automatic schedule splits
  // few pairs (partitions sized on those lengths, or unsplit where every
  // context fits one); otherwise the append kernel, then the decode.
  const int64_t pairs = pl.S * pl.Hkv * ((pl.Hq / pl.Hkv + 15) / 16);
  const bool mfma = pl.path == pa::Path::Mfma;
  const bool unsplit = !pl.stream && pl.max_parts == 1;
  const bool host_split = mfma && !unsplit && host_lens && opts->partition_tokens == 0 &&
                          (pl.stream || pairs < kFullGpuPairs);
  bool shared_unsplit = false;  // one or two q heads per KV head, a grid that fills the GPU
  if (unsplit && pl.share_unsplit) {
    int cus = 0;
    if ((rc = device_cus(&cus)) != PA_OK) return rc;
    shared_unsplit = pl.Hkv * pl.S >= cus;
  }
  if ((mfma && unsplit && !shared_unsplit) || host_split) {
    const CacheGeom g{pl.NB, pl.Hkv, pl.D, pl.B};
    pa::MultiParams m;
    if ((rc = multi_params(out, q, k, v, slot_mapping, nullptr, k_cache, v_cache, block_tables, context_lens,
                           g, scale, 1, &m)) != PA_OK)
      return rc;
    if (!host_split || !host_length_split(pl.S, pl.Hkv, pl.W * pl.B, host_lens, 1, &m) ||
        pa::workspace_layout(pl.S, pl.Hq, pl.D, m.d.max_parts).total <= workspace_bytes)
      return launch_fused_step(pl, &m, opts, workspace, stream);
  }
  if (!pl.stream && ((mfma && pl.max_parts > 1) || pl.share_unsplit)) {
    // partitioned: where the schedule runs the shared-partition kernel, it
    // takes the append too (its last partitions read the new token from k / v)
    const CacheGeom g{pl.NB, pl.Hkv, pl.D, pl.B};
    pa::MultiParams m;
    if ((rc = multi_params(out, q, k, v, slot_mapping, nullptr, k_cache, v_cache, block_tables, context_lens,
                           g, scale, 1, &m)) != PA_OK)
      return rc;
    m.d.head_groups = (m.d.group + 15) / 16;
    m.d.part_tokens = pl.part_tokens;
    m.d.max_parts = pl.max_parts;
    m.d.share_unsplit = pl.share_unsplit;
    int cus = 0;
    if ((rc = device_cus(&cus)) != PA_OK) return rc;
    const pa::LaunchCtx ctx{stream, opts ? opts->kernel_start : nullptr, opts ? opts->kernel_stop : nullptr,
                            cus, host_lens};
    if (pa::shared_step_applies(m.d, pl.path, ctx)) {
      if (m.d.max_parts > 1) {  // split: pieces in the workspace (unsplit rows are written directly)
        const pa::WorkspaceLayout wl = pa::workspace_layout(pl.S, pl.Hq, pl.D, m.d.max_parts);
        m.d.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
        m.d.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
      }
      const hipError_t e = pa::launch_shared_step(m, int(pl.D), int(pl.B), ctx);
      if (e != hipSuccess) return hip_fail(e, "fused append + shared-partition decode launch");
      return PA_OK;
    }
  }
  if ((rc = cache_append_impl(k, v, slot_mapping, k_cache, v_cache, false, stream)) != PA_OK) return rc;
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, opts, false,
                       workspace, workspace_bytes, false, stream);
}

PA_EXPORT int pa_copy_blocks(pa_tensor* k_cache, pa_tensor* v_cache, const pa_tensor* block_pairs,
                             hipStream_t stream) {
  begin_call();
  int rc;
  CacheGeom g;
  if ((rc = check_caches(k_cache, v_cache, &g)) != PA_OK) return rc;
  if ((rc = check_desc(block_pairs, "block_pairs", PA_I64, 2)) != PA_OK) return rc;
  const int64_t N = block_pairs->shape[0];
  if (block_pairs->shape[1] != 2)
    return fail(PA_ERR_INVALID, "block_pairs: shape [N, 2] expected, got [%lld, %lld]",
                (long long)N, (long long)block_pairs->shape[1]);
  if (N > 1 && (block_pairs->stride[0] != 2 || block_pairs->stride[1] != 1))
    return fail(PA_ERR_INVALID, "block_pairs must be contiguous");
  if (N == 0) return PA_OK;
  if (N > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "too many block pairs");

  if (g_debug.load()) {
    std::vector<int64_t> pairs;
    if ((rc = copy_to_host(&pairs, block_pairs->data, size_t(2 * N), stream)) != PA_OK) return rc;
    std::unordered_set<int64_t> srcs, dsts;
    for (int64_t i = 0; i < N; ++i) srcs.insert(pairs[size_t(2 * i)]);
    for (int64_t i = 0; i < N; ++i) {
      const int64_t s = pairs[size_t(2 * i)], d = pairs[size_t(2 * i + 1)];
      if (s < 0 || s >= g.num_blocks || d < 0 || d >= g.num_blocks)
        return fail(PA_ERR_CONTRACT, "block_pairs[%lld] = (%lld, %lld) outside [0, %lld)", (long long)i,
                    (long long)s, (long long)d, (long long)g.num_blocks);
      if (!dsts.insert(d).second)
        return fail(PA_ERR_CONTRACT, "block_pairs[%lld]: destination %lld repeats", (long long)i,
                    (long long)d);
      if (srcs.count(d))
        return fail(PA_ERR_CONTRACT, "block_pairs[%lld]: destination %lld is also a source",
                    (long long)i, (long long)d);
    }
  }

  pa::CopyParams p{};
  p.pairs = static_cast<const int64_t*>(block_pairs->data);
  p.k_cache = static_cast<uint16_t*>(k_cache->data);
  p.v_cache = static_cast<uint16_t*>(v_cache->data);
  p.num_blocks = g.num_blocks;
  p.block_units = g.kv_heads * g.block_size * g.head_dim * 2 / 16;
  p.num_pairs = int(N);
  const hipError_t e = pa::launch_copy(p, stream);
  if (e != hipSuccess) return hip_fail(e, "copy launch");
  return PA_OK;
}

PA_EXPORT int pa_cache_append(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping,
                              pa_tensor* k_cache, pa_tensor* v_cache, hipStream_t stream) {
  begin_call();
  return cache_append_impl(k, v, slot_mapping, k_cache, v_cache, g_debug.load() != 0, stream);
}

namespace pa {

void note_launch(const char* name) {
  if (!g_launch.empty()) g_launch += ' ';
  g_launch += name;
}

}  // namespace pa
