/*
 * pa.h -- C ABI of libpa: PagedAttention decode for AMD MI355X (gfx950).
 *
 * The operations, as the PagedAttention pages describe them:
 *
 *   pa_cache_append  writes each new token's K and V into the slot of the
 *                    block pool that the host block manager assigned to it
 *                    ("vLLM - PagedAttention" digest (hungchun0201), "Fused
 *                    CUDA Kernels", item 1: fused reshape and block write;
 *                    "PagedAttention from First Principles", section 2: the
 *                    cache is append-only).
 *   pa_decode        one query per sequence attends to the sequence's cached
 *                    tokens, reached through its block table, with an online
 *                    softmax across blocks ("PagedAttention from First
 *                    Principles", section 5; Equation 4 of the hungchun0201
 *                    digest, "Mathematical Formulation").  Long contexts are
 *                    split into partitions whose partial softmax results are
 *                    combined by a log-sum-exp reduce ("PagedAttention from
 *                    First Principles", section 17, the v2 kernel's reduce).
 *   pa_append_decode the append and the decode of a step in one call, one
 *                    launch where the schedule allows.
 *   pa_decode_multi  several new tokens per sequence (chunked prefill,
 *                    speculative verification): their append and their causal
 *                    attention in one launch.
 *   pa_decode_multi_ex, pa_decode_multi_workspace_bytes  the same with
 *                    options and the caller's workspace (no allocation).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor is device memory owned by the caller (for instance allocated
 *   by PyTorch) and described by a pa_tensor: element strides, not bytes.
 *   The library keeps no pointer after a call returns.
 * - Work is enqueued on `stream` (NULL = the default stream) and the call
 *   returns without waiting.  A status code covers argument validation and
 *   launch errors only; pa_last_error() gives the message.  No entry point
 *   throws, aborts or prints.
 * - Device-side contracts are preconditions that are checked only in debug
 *   mode (pa_set_debug): block-table entries read by a sequence lie in
 *   [0, num_blocks); 0 <= context_lens[s] <= table_width * block_size; the
 *   slots of one append call are distinct and lie in [-1, num_blocks*B).
 *
 * Cache layout (one pool per K and per V, per layer)
 * --------------------------------------------------
 *   k_cache: bf16 [num_blocks, num_kv_heads, head_dim/8, block_size, 8]
 *            token t, dim d of block b, head h at [b, h, d/8, t, d%8]
 *   v_cache: bf16 [num_blocks, num_kv_heads, block_size/4, head_dim, 4]
 *            token t, dim d of block b, head h at [b, h, t/4, d, t%4]
 *   Both fully contiguous.  One (block, head) tile is block_size*head_dim
 *   contiguous elements.  A slot is block*block_size + offset.
 *   Supported: head_dim in {64, 128}; block_size in {8, 16, 32}.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument: null pointer, shape, dtype, stride */
  PA_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim, block_size, path) */
  PA_ERR_HIP = -3,         /* a HIP runtime call failed */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or too small */
  PA_ERR_CONTRACT = -5     /* debug mode: a device-side precondition is violated */
};

/* element types */
enum { PA_BF16 = 1, PA_F32 = 2, PA_I32 = 3, PA_I64 = 4 };

#define PA_MAX_DIMS 5

typedef struct {
  void* data;                   /* device pointer (may be NULL only if numel == 0) */
  int32_t dtype;                /* PA_BF16, PA_F32, PA_I32, PA_I64 */
  int32_t ndim;                 /* 1 .. PA_MAX_DIMS */
  int64_t shape[PA_MAX_DIMS];
  int64_t stride[PA_MAX_DIMS];  /* in elements */
} pa_tensor;

/*
 * pa_cache_append -- slot-mapped write of this step's K/V into the pools.
 *
 *   k, v          bf16 [T, num_kv_heads, head_dim]; last dim contiguous, every
 *                 row 16-byte aligned (row strides multiple of 8 elements).
 *   slot_mapping  int64 [T]; token i goes to slot slot_mapping[i]
 *                 (block = slot / B, offset = slot % B); a negative slot skips
 *                 the token (padding).
 *   k_cache, v_cache  the pools, layout above; written in place.
 *
 * Bit-exact copy.  No other slot of the pools is touched.  T == 0 is a no-op.
 */
int pa_cache_append(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping,
                    pa_tensor* k_cache, pa_tensor* v_cache, hipStream_t stream);

/*
 * pa_copy_blocks -- the copies of copy-on-write, all of a step in one launch.
 *
 * Before a sequence writes into a block it shares with others, the block is
 * duplicated into a free one and only that sequence's table is repointed
 * ("vLLM - PagedAttention" digest, "Copy-on-Write Logic"; "Fused CUDA
 * Kernels", item 3: the pending copies are batched into one launch).
 *
 *   k_cache, v_cache  the pools (layout above); written in place.
 *   block_pairs   int64 [N, 2], contiguous; row i = (src, dst): block dst of
 *                 both pools (every head, every slot) becomes a copy of block src.
 *
 * Bit-exact copy.  Preconditions (checked in debug mode only): every id lies
 * in [0, num_blocks), destinations are distinct and none is also a source
 * (then the rows are independent and their order does not matter).  A row
 * naming a block outside the pool is skipped.  N == 0 is a no-op.
 */
int pa_copy_blocks(pa_tensor* k_cache, pa_tensor* v_cache, const pa_tensor* block_pairs,
                   hipStream_t stream);

/*
 * pa_decode -- paged decode attention, one query token per sequence.
 *
 *   out           bf16 (rounded to nearest even) or f32 [S, num_q_heads, head_dim],
 *                 last dim contiguous.
 *   q             bf16 [S, num_q_heads, head_dim], last dim contiguous.
 *   k_cache, v_cache  the pools (read only).
 *   block_tables  int32 [S, W]; row s lists the physical blocks of sequence s
 *                 in logical order; only the first ceil(L_s / B) entries are
 *                 read, the rest may hold any sentinel (-1 by convention).
 *   context_lens  int32 [S]; L_s tokens, this step's token included.
 *   scale         multiplies q.k (1/sqrt(head_dim) for standard attention).
 *   block_size    must equal the pools' block size.
 *
 * out[s, h, :] = softmax_t(scale * q[s,h,:] . K[s,t,:]) V[s,t,:] over t < L_s,
 * with query head h reading KV head h / (num_q_heads / num_kv_heads).  An empty
 * context (L_s == 0) yields zeros.  Tokens at t >= L_s are never read, so
 * their values (even NaN) cannot affect the result.  bf16 products, fp32
 * accumulation; results are bitwise deterministic.
 *
 * Schedule, chosen from the shapes alone (P = num_seqs * num_kv_heads *
 * ceil(G / 16) pairs, G = q heads per KV head, Lmax = table width *
 * block_size):
 *   P >= 512, G >= 3, Lmax <= 8192  one workgroup per pair, no split;
 *   P >= 512 otherwise              partitions of 1024 tokens;
 *   Lmax <= 1024                    one workgroup per pair (short tables);
 *   P * ceil(Lmax / 512) <= 2048    partitions of 512 tokens (few pairs with
 *                                   long tables: the grid still fits the GPU
 *                                   about once, so the partitions a shorter
 *                                   context leaves empty cost little);
 *   otherwise                       stream-K: the 16-token tiles of all pairs
 *                                   are cut into equal contiguous ranges, one
 *                                   per wave of a persistent grid, and a
 *                                   context is split where a cut falls
 *                                   (batches of more than 8192 sequences:
 *                                   partitions of 512 tokens).
 * A second kernel combines the partial results of a split context in
 * ascending token order with a log-sum-exp reduce.  Blocks that consecutive
 * sequences hold in common (a shared prefix, "PagedAttention from First
 * Principles", section 9) are read once for a run of up to 16/G of them, by
 * the shared-partition kernel: under partitions with G <= 16, and on the
 * automatic unsplit schedule with G <= 2, wherever the grid holds a
 * workgroup per compute unit.  Within
 * a partition a run reads the members' common leading blocks once, then each
 * member's own; it grows member by member while the own 16-token tiles do
 * not outnumber the common ones.  Keep sequences that share a prefix
 * adjacent; the results do not depend on it.  The partial results live in a
 * library-owned workspace on the current device, grown with hipMalloc when a
 * call needs more (never during stream capture: that returns PA_ERR_WORKSPACE;
 * use pa_decode_ex there).  Calls that need the workspace may not overlap on
 * one device from different host threads unless they are on the same stream.
 */
int pa_decode(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
              const pa_tensor* v_cache, const pa_tensor* block_tables,
              const pa_tensor* context_lens, float scale, int32_t block_size,
              hipStream_t stream);

/* options for pa_decode_ex; a zero-initialised struct means "as pa_decode" */
typedef struct {
  int32_t partition_tokens;  /* 0: automatic, from the shapes (see pa_decode);
                                -1: one partition per sequence (never split);
                                -2: the stream-K schedule;
                                else partitions of this many tokens, a positive
                                multiple of 32 */
  int32_t path;              /* 0: auto (the MFMA path);
                                1: the VALU path (q heads per KV head <= 2);
                                2: the MFMA path */
  int64_t max_context_len;   /* partitioned schedule only.  0: table width *
                                block_size; else an upper bound on every
                                context_lens[s], used to size the launch */
  int32_t workgroups_per_cu; /* stream-K schedule only: persistent workgroups
                                per compute unit, 0 = default (2), at most 64 */
  int32_t reserved;          /* must be 0 */
  hipEvent_t kernel_start;   /* both NULL, or both events created by the caller:  */
  hipEvent_t kernel_stop;    /* they then record the start and the end of the
                                main decode kernel alone (not the combine), as
                                timed by the GPU (hipExtLaunchKernel) */
  const int32_t* host_context_lens; /* NULL, or HOST memory holding a copy of
                                context_lens ([num_seqs] int32), read during
                                the call only; it must equal the device's
                                lengths (a precondition, reported as
                                PA_ERR_CONTRACT under pa_set_debug(1)).
                                Where max_context_len is 0, the longest of
                                them bounds the launch in its place (tables
                                are often sized for a model's maximum context).
                                Unsplit schedules then rank the sequences on
                                the host and pass the order with the kernel's
                                arguments, instead of every workgroup loading
                                and ranking the lengths first; there it steers
                                only placement, and results are identical with
                                or without it.  pa_append_decode also uses it
                                where the automatic schedule splits with few
                                pairs (MFMA path): partitions sized on the
                                lengths so that the workgroups share the tokens
                                evenly, only those holding tokens launched, the
                                append fused into that launch */
} pa_decode_opts;

/* Bytes of workspace pa_decode_ex needs for these sizes (0 when nothing is split). */
size_t pa_decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                                 int64_t head_dim, int64_t max_context_len,
                                 int32_t partition_tokens);

/*
 * The schedule an automatic call (pa_decode, or pa_decode_ex with
 * partition_tokens 0) takes for these sizes, where max_context_len is the
 * table width times block_size (or opts.max_context_len): *partition_tokens
 * receives -1 (no split), -2 (stream-K) or the partition size in tokens.
 * Returns PA_OK, or PA_ERR_INVALID for a NULL pointer, negative sizes or
 * num_q_heads not a multiple of num_kv_heads.  Host only; launches nothing.
 */
int pa_decode_schedule(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                       int64_t max_context_len, int32_t* partition_tokens);

/*
 * pa_decode_ex -- pa_decode with options and a caller-owned workspace.
 *
 * `workspace` is device memory of at least pa_decode_workspace_bytes(...)
 * bytes, 256-byte aligned, with any contents (it only carries partial results
 * from the decode kernel to the combine kernel of the same call).  It must not
 * be shared by calls that may run concurrently.  Nothing is allocated, so the
 * call may be captured into a HIP graph.  workspace may be NULL when the
 * required size is 0.
 */
int pa_decode_ex(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                 const pa_tensor* v_cache, const pa_tensor* block_tables,
                 const pa_tensor* context_lens, float scale, int32_t block_size,
                 const pa_decode_opts* opts, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Bytes of device memory the library reserves, once per GPU it runs on, for
 * pa_decode_noalloc's partial results (held until the process ends). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.
 *
 * Arguments, schedule, preconditions and results are pa_decode's; the outputs
 * equal pa_decode's bit for bit.  A split schedule keeps its partial results
 * (the only memory beyond the inputs and outputs) in a fixed array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds per GPU, instead of
 * pa_decode's growable workspace.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its first call on a device looks up
 * that device's copy of the array.
 *
 * A call whose schedule needs more than PA_NOALLOC_SCRATCH_BYTES
 * (pa_decode_workspace_bytes with max_context_len = table width * block_size
 * and partition_tokens 0) returns PA_ERR_WORKSPACE before launching anything;
 * use pa_decode_ex with a workspace of that size instead.  Every call on a GPU
 * shares that GPU's array, and a call does not depend on what an earlier one
 * left in it (each split call writes every entry before its combine reads
 * it).  Calls that may overlap on one GPU (different streams, or different
 * host threads without ordering) race on the array: order them on one
 * stream.
 */
int pa_decode_noalloc(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache,
                      const pa_tensor* v_cache, const pa_tensor* block_tables,
                      const pa_tensor* context_lens, float scale, int32_t block_size,
                      hipStream_t stream);

/*
 * pa_decode_contiguous -- the control for paging: the same decode over a cache
 * that is not paged.
 *
 * The pages report that table lookups and variable lengths made the paper's
 * paged kernel 20-26 % slower than an optimized contiguous one (chenyuan1125
 * essay, "The Block Table Separates Logical from Physical Contiguity";
 * "PagedAttention Explained" (sevydevy), its list of costs).  This entry
 * point measures that cost for this library: each (sequence, KV head) owns
 * one contiguous run of max_len/16 tiles of 16 tokens, each tile in the format
 * of a 16-token block of one head, and the kernel is pa_decode's MFMA kernel
 * with the tile address computed instead of looked up.
 *
 *   out, q        as for pa_decode.
 *   k             bf16 [S*Hkv, max_len/16, D/8, 16, 8]: token t, dim d of
 *                 sequence s, head h at [s*Hkv + h, t/16, d/8, t%16, d%8];
 *                 contiguous.
 *   v             bf16 [S*Hkv, max_len/16, 4, D, 4]: at [s*Hkv + h, t/16,
 *                 (t%16)/4, d, t%4]; contiguous.
 *   context_lens  int32 [S]; tokens t < L_s are read (L_s > max_len is clamped).
 *   scale         as for pa_decode.
 *
 * max_len * D * 2 < 2^31; head_dim 64 or 128; any query-head grouping (MFMA
 * path); no split, no workspace.  The result equals pa_decode's unsplit MFMA
 * schedule on the same values, bit for bit.
 */
int pa_decode_contiguous(pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                         const pa_tensor* context_lens, float scale, hipStream_t stream);

/*
 * pa_append_decode -- one decode step in one call: this step's K/V appended
 * at their slots, then pa_decode_ex over the updated pools.
 *
 * The append and the attention are the two halves of a decode step ("vLLM -
 * PagedAttention" digest, "Fused CUDA Kernels": the write into the cache is
 * fused to cut launches; "PagedAttention from First Principles", section 5).
 * Where the decode schedule is unsplit on the MFMA path (but for the grids of
 * one or two q heads per KV head that the shared-partition kernel takes,
 * below), one kernel does both:
 * it stores the new token and takes its K/V from k / v for the attention.
 * Where the automatic schedule splits with fewer than 512 pairs (stream-K or
 * 512-token partitions) and opts carries host_context_lens, the multi-token
 * kernel does both over partitions sized on those lengths (in the workspace),
 * and a second kernel combines each row's partitions; where those lengths
 * fit one partition each, the unsplit fused kernel runs.  Where the
 * schedule is partitioned on the MFMA path (grouping <= 16), or unsplit with
 * grouping <= 2, and the grid fills the GPU, the step takes two launches
 * instead of three: the workgroup
 * of a sequence's last partition in the shared-partition kernel reads the
 * pool up to the new position and folds the new token in from k / v, and the
 * combine kernel that follows also stores the new tokens.  Otherwise the
 * append kernel runs, then the decode the schedule chooses (outputs then
 * equal the two calls' bit for bit; the fused kernels differ from them only
 * in rounding).
 *
 *   out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
 *   opts, workspace, workspace_bytes: as for pa_decode_ex (kernel events in
 *                 opts time the fused kernel, or the main decode kernel).
 *   k, v          bf16 [S, num_kv_heads, head_dim]: sequence s's new token,
 *                 its position L_s - 1; last dim contiguous, rows 16-byte aligned.
 *   slot_mapping  int64 [S]: the slot of that position.
 *
 * The result equals pa_cache_append followed by pa_decode_ex with the same
 * options, up to rounding where a fused kernel runs or host lengths pick the
 * partitions.  Preconditions (debug mode checks them, with pa_decode's): for
 * every sequence with L_s > 0, slot_mapping[s] is the slot its block table
 * gives position L_s - 1; a sequence with L_s == 0 has no new token and a
 * negative slot; no sequence reads a slot that receives another sequence's
 * new token (copy-on-write has made the block that receives a new token
 * private to its sequence; the fused kernels read the pools before the new
 * tokens are stored, the two calls after).  Every argument, the workspace
 * included, is checked before anything is launched.  S == 0 is a no-op.
 */
int pa_append_decode(pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                     const pa_tensor* slot_mapping, pa_tensor* k_cache, pa_tensor* v_cache,
                     const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                     int32_t block_size, const pa_decode_opts* opts, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_multi -- several new tokens per sequence in one step: the append
 * and the attention of chunked prefill and of speculative verification.
 *
 * A prefill split into chunks brings a chunk of a prompt in one scheduler step
 * beside other sequences' single decode tokens ("PagedAttention from First
 * Principles", section 12); a verifier checks the draft's tokens of every
 * sequence in one pass and appends them to its cache ("PagedAttention from
 * First Principles", section 14).  Sequence s brings n_s = query_start[s+1] -
 * query_start[s] tokens, which are its positions L_s - n_s .. L_s - 1.
 *
 *   out           bf16 or f32 [T, num_q_heads, head_dim], last dim contiguous;
 *                 row r belongs to the new token in row r of q.
 *   q             bf16 [T, num_q_heads, head_dim]; rows query_start[s] ..
 *                 query_start[s+1]-1 are sequence s's new tokens in order.
 *   k_new, v_new  bf16 [T, num_kv_heads, head_dim]: their keys and values.
 *                 q, k_new, v_new: last dim contiguous, rows 16-byte aligned.
 *   slot_mapping  int64 [T]: the slot of each new token; a negative slot
 *                 skips the store (the token still takes part in attention).
 *   query_start   int32 [S + 1], non-decreasing, query_start[S] <= T.
 *   k_cache, v_cache  the pools (layout above): the new tokens are written,
 *                 nothing else is touched.
 *   block_tables, context_lens, scale, block_size  as for pa_decode; L_s
 *                 counts the new tokens.
 *   max_query_len an upper bound on n_s (the launch covers that many rows per
 *                 sequence); max_query_len * (num_q_heads / num_kv_heads) <= 2^24.
 *
 * New token i of sequence s (row r = query_start[s] + i) attends to the
 * positions 0 .. L_s - n_s + i: the cached ones and the new ones up to itself.
 * out[r, h, :] = softmax_t(scale * q[r,h,:] . K[s,t,:]) V[s,t,:] over those t,
 * with K and V of the new positions taken from k_new / v_new (equal to what
 * the store puts in the pools).  Same arithmetic as pa_decode.  Preconditions
 * (debug mode checks them): 0 <= n_s <= min(L_s, max_query_len); each
 * non-negative slot is the table's slot for its position and no slot repeats;
 * no cached position read by the call (t < L_s - n_s of any sequence) lies in
 * a slot it writes.  Rows outside every sequence's range are not written; a
 * sequence's rows past its context length (n_s > L_s) are written as zeros.
 * S == 0, T == 0 or max_query_len == 0 is a no-op.  With few sequences the
 * cached context is split into partitions joined by a log-sum-exp combine, in
 * the library-owned workspace of pa_decode (same growth and threading rules).
 */
int pa_decode_multi(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_new, const pa_tensor* v_new,
                    const pa_tensor* slot_mapping, const pa_tensor* query_start, pa_tensor* k_cache,
                    pa_tensor* v_cache, const pa_tensor* block_tables, const pa_tensor* context_lens,
                    float scale, int32_t block_size, int32_t max_query_len, hipStream_t stream);

/*
 * pa_decode_multi_ex -- pa_decode_multi with options and the caller's
 * workspace: it allocates nothing, so it may be captured into a HIP graph.
 *
 *   opts          NULL (as pa_decode_multi) or pa_decode_opts:
 *                   partition_tokens  0 automatic (as pa_decode_multi), -1
 *                                     never split, else partitions of this
 *                                     many cached tokens (a positive multiple
 *                                     of 32); -2 (stream-K) is
 *                                     PA_ERR_UNSUPPORTED here;
 *                   path              0 or 2 (the multi-token kernels are
 *                                     MFMA only; 1 is PA_ERR_UNSUPPORTED);
 *                   max_context_len   0, or a bound on every context_lens[s]
 *                                     that sizes a split;
 *                   workgroups_per_cu, reserved  must be 0;
 *                   kernel_start, kernel_stop  as for pa_decode_ex (the main
 *                                     kernel, not the combine);
 *                   host_context_lens as for pa_decode_ex: unsplit launches
 *                                     rank the sequences on the host; an
 *                                     automatic split with few pairs is sized
 *                                     on them, launching only the partitions
 *                                     that hold tokens (within the workspace
 *                                     given; else the shape-only split), and
 *                                     where max_context_len is 0 the longest
 *                                     of them bounds a split.
 *   workspace, workspace_bytes  device memory, 256-byte aligned, of at least
 *                 pa_decode_multi_workspace_bytes(T, num_seqs, num_q_heads,
 *                 num_kv_heads, head_dim, max_query_len, bound,
 *                 opts->partition_tokens) bytes, bound being the split's
 *                 bound above (or anything larger); NULL / 0 when that is 0.
 *                 PA_ERR_WORKSPACE if too small or misaligned.  Calls that
 *                 share a workspace must be ordered on one stream.
 *
 * Everything else (arguments, preconditions, results) is pa_decode_multi's;
 * with the same split the two give identical bits.
 */
int pa_decode_multi_ex(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_new, const pa_tensor* v_new,
                       const pa_tensor* slot_mapping, const pa_tensor* query_start, pa_tensor* k_cache,
                       pa_tensor* v_cache, const pa_tensor* block_tables, const pa_tensor* context_lens,
                       float scale, int32_t block_size, int32_t max_query_len, const pa_decode_opts* opts,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes pa_decode_multi_ex needs for num_rows (T) new tokens of
 * num_seqs sequences, max_query_len rows per sequence at most, cached
 * contexts bounded by max_context_len, and opts.partition_tokens as given
 * (0 = automatic).  0 when the launch does not split (or for sizes <= 0). */
size_t pa_decode_multi_workspace_bytes(int64_t num_rows, int64_t num_seqs, int64_t num_q_heads,
                                       int64_t num_kv_heads, int64_t head_dim, int32_t max_query_len,
                                       int64_t max_context_len, int32_t partition_tokens);

/* Message of the last failed call on this thread (valid until the next pa_* call). */
const char* pa_last_error(void);

/*
 * The kernels the last call of an entry point that takes a stream enqueued on
 * this thread, in launch order, separated by spaces, each as its template
 * instantiation (for instance "decode_shared<128,16,true> combine_append<128,16>");
 * empty if it launched nothing.  For tests and benchmarks that need to know
 * which schedule ran.  Valid until the next pa_* call on this thread.
 */
const char* pa_last_launch(void);

/*
 * Debug mode (process-wide, off by default).  When on, the entry points that
 * take index tensors (appends, copies, paged decodes) copy them to the host,
 * synchronise `stream`, and check the device-side contracts listed above and
 * at each entry point before launching; a violation returns PA_ERR_CONTRACT.
 * Returns the previous setting.
 */
int pa_set_debug(int on);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
