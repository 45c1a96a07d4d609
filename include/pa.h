/*
 * pa.h -- C ABI of libpa: paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * Sources (the web pages the method is taken from; cited below by tag and section):
 *   [P1] "PagedAttention", inferensys.com glossary entry
 *   [P2] "Paged Attention" tutorial, infra.pidoku.co.in (inference engineering, vLLM, file 10)
 *   [P4] "PagedAttention & KV-Cache Management in High-Throughput LLM Serving",
 *        subroutine-cs.cc
 *
 * Conventions for every entry point
 *   - Device pointers are owned by the caller (allocated through any HIP allocator; the
 *     library never allocates device memory). Host pointers are read during the call only.
 *   - Tensors are dense, row-major, with the shapes given. Cache base pointers and q must
 *     be 16-byte aligned; block_tables, seq_lens and slot_mapping 4-byte aligned.
 *   - Cache layout, K and V alike: [num_blocks, num_kv_heads, block_size, head_dim]. Each
 *     (physical block, KV head) is one contiguous [block_size, head_dim] tile.
 *   - Element types (kv_dtype): PA_F32 (IEEE binary32) or PA_BF16 (bfloat16, 16 raw bits).
 *   - stream is a hipStream_t passed as void* (NULL = the null stream). Kernel entry points
 *     are asynchronous: they validate, enqueue and return.
 *   - Return value: PA_OK or a negative PA_ERR_* code. Argument checks are pure host code
 *     and run before any HIP call; on an error nothing is enqueued and pa_last_error()
 *     describes it (thread-local). Device-resident data (table entries, lengths, slots)
 *     is not read on the host: entries outside their documented range give unspecified
 *     results for the rows they touch but never an access outside the buffers.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 2

/* element types */
#define PA_F32 0
#define PA_BF16 1

/* decode work decompositions (pa_set_decode_path) */
#define PA_PATH_AUTO 0
#define PA_PATH_PARTITION 1
#define PA_PATH_STREAM 2

/* status codes */
#define PA_OK 0
#define PA_ERR_INVALID_ARG (-1) /* null pointer, bad shape, misalignment, small workspace */
#define PA_ERR_UNSUPPORTED (-2) /* valid but not built: head_dim, block_size, group size */
#define PA_ERR_NO_BLOCKS (-3)   /* allocator: not enough free blocks */
#define PA_ERR_HIP (-4)         /* the HIP runtime reported an error at launch */

/* ------------------------------------------------------------------ decode attention */

/*
 * pa_decode -- paged decode attention over a ragged batch ([P1] "Interpret Block Tables"
 * and "Handle Variable-Length Sequences"; [P2] section 5 "The kernel side"; [P4] section 1,
 * the decode phase).
 *
 * For sequence b and query head h, with G = Hq / Hkv and KV head g = h / G (consecutive
 * query heads share a KV head) and L = seq_lens[b]:
 *   token t < L is read from physical block block_tables[b][t / block_size], slot
 *   t % block_size;  s_t = scale * <q[b,h,:], K_t>;  out[b,h,:] = sum_t softmax(s)_t V_t.
 * L == 0 gives out[b,h,:] = 0. Slots past L in the last block and table entries past
 * ceil(L / block_size) are never read.
 *
 *   out           device float [B, Hq, D] (always fp32)
 *   q             device [B, Hq, D], element type kv_dtype
 *   k_cache       device [num_blocks, Hkv, block_size, D]
 *   v_cache       device, same shape and type as k_cache
 *   block_tables  device int32 [B, max_blocks]; entries j < ceil(L_b / block_size) must
 *                 lie in [0, num_blocks)
 *   seq_lens      device int32 [B]; 0 <= L_b <= max_blocks * block_size
 *   scale         softmax scale, applied in fp32 to the fp32 dot product
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...) bytes, 256-byte
 *                 aligned (may be NULL when that size is 0); it holds partial softmax
 *                 states of sequences split across work items and needs no
 *                 initialisation. Calls that share one workspace must not overlap.
 * Supported: D in {64, 128}; block_size in {8, 16, 32, 64, 128} (8 with bf16 caches and
 * the stream decomposition only); G in {1, 2, 4, 8}; B <= 65535; others, and batches with
 * more work items or merged rows (B x Hq) than one launch grid holds, return
 * PA_ERR_UNSUPPORTED. The result is deterministic: repeated calls on one device give
 * identical bits, whatever the physical placement of the blocks.
 *
 * Work decomposition (chosen per call, see pa_set_decode_path):
 *   stream     (bf16 caches, B <= 4096, fewer than 2^31 groups of 16 tokens in the batch):
 *              the batch's (sequence, KV head) rows, cut into 16-token groups, are laid
 *              end to end and every resident wavefront of the device takes an equal
 *              contiguous slice; rows that cross slices are merged, in a fixed order, by
 *              a second kernel.
 *   partition  (otherwise): one work item per (sequence, KV head, partition of
 *              pa_decode_partition_tokens tokens), then a merge of the partitions.
 */
int32_t pa_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                  int32_t max_blocks, float scale, int32_t kv_dtype, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Workspace bytes pa_decode needs for these sizes and element type with the decomposition
 * it picks under the current pa_set_decode_path setting (0 when it needs none); an upper
 * bound from the host-known max_blocks. Returns 0 for sizes pa_decode would reject. A
 * change of the path, partition or wave settings changes the size: query it again.
 *   Hkv and kv_dtype are needed because the decomposition depends on them: bf16 caches
 *   take the stream decomposition, whose partial records hold the G = Hq / Hkv query
 *   heads of a KV head, two per wavefront that gets a slice: 2 x ns x G x (D + 2) x 4
 *   bytes plus 16 bytes per launched wavefront nw. nw is the number of wavefronts the
 *   current device holds at once (4096 when no device is visible); ns <= nw is no more
 *   than the batch fills with 8 groups of 16 tokens each (pa_set_stream_waves changes
 *   both).
 *   fp32 caches take the partition decomposition: B x Hq x n_parts x (D + 2) x 4 bytes when
 *   a sequence can span more than one partition of pa_decode_partition_tokens tokens, else 0.
 * The size depends on the current device; allocate it on the device the calls run on.
 */
size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                 int32_t max_blocks, int32_t kv_dtype);

/*
 * pa_decode_append -- one decode step in one launch: the cache write of each sequence's
 * newest token (pa_reshape_and_cache with T = B) and pa_decode over the batch that
 * includes it ([P4] section 1, the decode phase: each new token's K/V joins the cache and
 * the token attends to it; reading [P4] section 1 as in pa_decode, position L_b - 1 is the
 * newest token and is attended).
 *
 *   key, value    device [B, Hkv, D], kv_dtype: the newest token's K and V rows
 *   slot_mapping  device int32 [B]: the slot of sequence b's newest token, i.e. the slot
 *                 of its position seq_lens[b] - 1 (table[(L-1) / bs] * bs + (L-1) % bs),
 *                 or < 0 for a sequence with no new token (its position L - 1 is then
 *                 read from the cache); distinct
 *   k_cache, v_cache are written (the given slots) and read
 * Every other argument, the workspace and the errors as for pa_decode. The result, caches
 * and output alike, is that of pa_reshape_and_cache followed by pa_decode: on the stream
 * decomposition one launch writes the rows and reads position L - 1 from key / value, so no
 * wavefront reads a slot written in the same launch; otherwise the cache write is its own
 * kernel, launched first. A slot that breaks the precondition gives wrong rows for its
 * sequence (the debug validation pass reports it as PA_BAD_APPEND_SLOT).
 */
int32_t pa_decode_append(float* out, const void* q, void* k_cache, void* v_cache, const void* key,
                         const void* value, const int32_t* slot_mapping, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks, float scale,
                         int32_t kv_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). It allocates nothing either: the partial softmax states live in
 * a scratch array of 16 MiB that the library holds on each device until the process ends
 * (its address is looked up on the first call on a device). Arguments, results and errors
 * as for pa_decode; sizes whose pa_decode_workspace_bytes exceeds 16 MiB return
 * PA_ERR_INVALID_ARG (use pa_decode with a workspace). Every call on one device shares
 * that device's scratch, so calls that overlap on one device (several streams or host
 * threads) race: serialise them. The scratch needs no initialisation.
 */
int32_t pa_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks, float scale, int32_t kv_dtype, void* stream);

/*
 * Tokens per partition that pa_decode uses for these sizes (a sequence longer than this
 * is split into partitions whose partial softmax results are combined exactly).
 */
int32_t pa_decode_partition_tokens(int32_t block_size, int32_t max_blocks);

/*
 * Process-wide override of the partition length, for tuning sweeps and tests: tokens must
 * be 0 (automatic) or a multiple of 64 in [64, 1024]. Not thread-safe; affects calls made
 * after it returns, including pa_decode_workspace_bytes.
 */
int32_t pa_set_partition_tokens(int32_t tokens);

/*
 * Process-wide choice of decomposition, for tests and sweeps: PA_PATH_AUTO (default:
 * stream where it applies, else partition), PA_PATH_PARTITION, or PA_PATH_STREAM (then
 * pa_decode returns PA_ERR_UNSUPPORTED where the stream decomposition does not apply).
 * Not thread-safe.
 */
int32_t pa_set_decode_path(int32_t path);

/*
 * Process-wide stream decomposition settings, for tests and sweeps: waves in [0, 4096]
 * (0 = every wavefront the device holds at once, else that many, rounded up to a
 * multiple of 4) and min_slice in [0, 2^20] (0 = default 8): fewer waves are used when
 * slices would hold fewer than min_slice groups of 16 tokens. Not thread-safe.
 */
int32_t pa_set_stream_waves(int32_t waves, int32_t min_slice);

/*
 * Process-wide order in which pa_decode_multi's query-tile work is handed to the waves,
 * for tests and sweeps: 1 (default) longest first, 0 the plain grid order (KV head, tile
 * from the last, partition, sequence). The order changes only which wavefront runs which
 * piece of work, never the result: both give identical bits. Not thread-safe.
 */
int32_t pa_set_multi_order(int32_t longest_first);

/*
 * pa_decode_shared -- pa_decode for a batch in which groups of consecutive sequences
 * share their leading blocks (shared prompts and parallel sampling: [P1] "Shared Prompts"
 * and "Parallel Sampling"; [P2] section 5 "Copy-on-write sharing"). Every shared K/V tile
 * is read from HBM once for all members of its group instead of once per member; the
 * result equals pa_decode's up to rounding.
 *
 *   groups             device int32 [n_groups, 3]: first sequence, members, shared tokens.
 *                      Members are sequences first .. first + members - 1; groups are
 *                      sorted by first sequence and disjoint. For every member, the table
 *                      entries covering the shared tokens equal the first member's, and
 *                      seq_lens >= shared tokens. Shared tokens are used rounded down to a
 *                      multiple of 16 (the tokens past that are read per member).
 *   n_groups           host count of groups (0: every sequence is read on its own)
 *   max_members        host bound on the members of any group; max_members * Hq / Hkv
 *                      must not exceed 64
 *   max_shared_tokens  host bound on any group's shared tokens (<= max_blocks * block_size)
 *   workspace          at least pa_decode_shared_workspace_bytes(...) bytes, 256-byte
 *                      aligned; needs no initialisation
 * bf16 caches, block_size in {16, 32, 64, 128}; every other argument as for pa_decode.
 * Violated group preconditions give wrong rows for the sequences concerned, never an
 * access outside the buffers.
 */
int32_t pa_decode_shared(float* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* groups, int32_t n_groups, int32_t max_members,
                         int32_t max_shared_tokens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks, float scale,
                         int32_t kv_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pa_decode_shared needs (0 for sizes it would reject). */
size_t pa_decode_shared_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t block_size,
                                        int32_t max_blocks, int32_t max_shared_tokens);

/*
 * pa_decode_multi -- several of each sequence's newest tokens attend at once, with a
 * causal mask: the prompt of the prefill phase ([P4] section 1: all prompt tokens in
 * parallel), a later chunk of a long prompt, or draft tokens checked in one pass. The
 * decode step of pa_decode is the case of one query per sequence.
 *
 * The chunk's keys and values must already be in the cache (pa_reshape_and_cache at
 * their slots). Sequence b's queries are the last n_b = q_starts[b+1] - q_starts[b] of
 * its seq_lens[b] tokens, in position order: query j (global row q_starts[b] + j) sits at
 * position p = seq_lens[b] - n_b + j and attends to tokens 0 .. p, its own included.
 *
 *   out        device fp32 [total_q, Hq, D], written
 *   q          device [total_q, Hq, D], the cache's element type
 *   q_starts   device int32 [B + 1]: q_starts[0] = 0, non-decreasing, q_starts[B] = total_q,
 *              0 <= n_b <= min(seq_lens[b], max_q)
 *   total_q    host count of query tokens
 *   max_q      host bound on any n_b (it sizes the query tiles)
 *   workspace  pa_decode_multi_workspace_bytes(...) bytes, 256-byte aligned, needs no
 *              initialisation; may be NULL when that size is 0 (no token split)
 * bf16 caches, block_size in {16, 32, 64, 128}, head_dim in {64, 128}, any Hq / Hkv;
 * every other argument as for pa_decode. Offsets that break the preconditions are clamped
 * on the device: wrong rows for the sequences concerned, never an access outside the
 * buffers. Rows of queries no sequence owns are left unwritten.
 *
 * Chunks that fit one 16-column score tile per (sequence, KV head) (max_q x Hq / Hkv <= 16,
 * e.g. draft tokens) run on pa_decode's stream decomposition. Longer ones are cut into
 * query tiles of up to 64 rows; the tiles see different numbers of tokens (a chunk's
 * later tiles more, a sequence with more cached tokens more), and the waves take them
 * longest first (for B <= 2048; pa_set_multi_order).
 */
int32_t pa_decode_multi(float* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* q_starts, int32_t B, int32_t total_q, int32_t max_q,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks, float scale, int32_t kv_dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes pa_decode_multi needs: 0 when it does not split any query's tokens
 * (or for sizes it would reject). */
size_t pa_decode_multi_workspace_bytes(int32_t B, int32_t total_q, int32_t max_q, int32_t Hq,
                                       int32_t Hkv, int32_t D, int32_t block_size,
                                       int32_t max_blocks);

/* ------------------------------------------------------------------ cache write */

/*
 * pa_reshape_and_cache -- write new tokens' K and V into their physical slots. Slot s is
 * the flat index table[pos / block_size] * block_size + pos % block_size of [P2] section 4
 * (PhysicalIndex); the row goes to block s / block_size, offset s % block_size. A bit copy.
 *
 *   k_cache, v_cache  device [num_blocks, Hkv, block_size, D], written
 *   key, value        device [T, Hkv, D]
 *   slot_mapping      device int32 [T]; s < 0 skips the token (padding); non-negative slots
 *                     must be distinct; slots >= num_blocks * block_size are skipped
 * T == 0 is a no-op. Supported: D a multiple of 8 (bf16) or 4 (fp32), up to 512.
 */
int32_t pa_reshape_and_cache(void* k_cache, void* v_cache, const void* key, const void* value,
                             const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                             int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                             void* stream);

/* ------------------------------------------------------------------ copy-on-write clone */

/*
 * pa_copy_blocks -- copy whole physical blocks, K and V, all heads and slots: the clone
 * taken before writing into a shared block ([P2] section 5 "Copy-on-write sharing"; [P4]
 * section 3). A bit copy.
 *
 *   block_pairs  device int32 [N, 2] of (src, dst); destinations must be distinct and no
 *                destination may also be a source, so the order of the copies is
 *                irrelevant; a pair with an index outside [0, num_blocks) is skipped
 * N == 0 is a no-op.
 */
int32_t pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t N,
                       int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                       int32_t kv_dtype, void* stream);

/* ------------------------------------------------------------------ debug validation */

/*
 * The kernels read device-resident indices without checking them against the
 * preconditions stated above (they clamp what they read, so a violation never reaches
 * outside the buffers, but the rows it touches come out wrong and nothing reports it).
 * The debug validation pass checks them: a table entry for each of a sequence's
 * ceil(L / block_size) logical blocks ([P1] "Interpret Block Tables"; [P2] section 4
 * "Tiny example", PhysicalIndex), one slot per new token, and copy-on-write clones into
 * fresh blocks that are then written ([P2] section 5 "Copy-on-write sharing": copy first,
 * then write), i.e. distinct destinations none of which another pair copies from.
 *
 * Flags of a validation (bitwise OR of every kind found):
 */
#define PA_BAD_LENGTH 0x1         /* seq_lens[b] outside [0, max_blocks * block_size] */
#define PA_BAD_TABLE_ENTRY 0x2    /* block_tables[b][j], j < ceil(L_b / block_size), outside [0, num_blocks) */
#define PA_BAD_SLOT 0x4           /* slot_mapping[i] >= num_blocks * block_size */
#define PA_DUP_SLOT 0x8           /* two tokens name the same non-negative slot */
#define PA_BAD_PAIR 0x10          /* a block_pairs index outside [0, num_blocks) */
#define PA_DUP_DST 0x20           /* two pairs copy into the same block */
#define PA_DST_IS_SRC 0x40        /* a destination block is also some pair's source */
#define PA_BAD_GROUP 0x80         /* pa_decode_shared groups break their preconditions */
#define PA_BAD_QUERY_STARTS 0x100 /* pa_decode_multi q_starts break their preconditions */
#define PA_BAD_APPEND_SLOT 0x200  /* pa_decode_append: a given slot is not where position L_b - 1 lives */

/*
 * Debug mode, process-wide (default off; PA_VALIDATE=1 in the environment when the
 * library first checks turns it on): every kernel entry point first copies its index
 * arrays (tables, lengths, slots, pairs, groups, query offsets) to the host on its own
 * stream, waits for them, and checks them; on a violation it returns PA_ERR_INVALID_ARG,
 * pa_last_error() names the first one, and nothing is enqueued. The calls then block the
 * host: for debugging, not for timing. pa_set_validation(on) takes 0 or 1.
 */
int32_t pa_set_validation(int32_t on);
int32_t pa_validation_enabled(void);

/*
 * Host validators (host pointers; the same checks the debug mode runs). Each returns
 * PA_OK, or PA_ERR_INVALID_ARG with pa_last_error() naming the first violation; *flags
 * (nullable) receives the PA_BAD_* / PA_DUP_* flags of all of them. Shapes as for the
 * kernel entry points; groups as for pa_decode_shared, q_starts as for pa_decode_multi.
 */
int32_t pa_validate_decode(const int32_t* block_tables, const int32_t* seq_lens, int32_t B,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks,
                           uint32_t* flags);
int32_t pa_validate_slots(const int32_t* slot_mapping, int32_t T, int32_t block_size,
                          int32_t num_blocks, uint32_t* flags);
int32_t pa_validate_block_pairs(const int32_t* block_pairs, int32_t N, int32_t num_blocks,
                                uint32_t* flags);
int32_t pa_validate_groups(const int32_t* groups, int32_t n_groups, const int32_t* block_tables,
                           const int32_t* seq_lens, int32_t B, int32_t block_size,
                           int32_t max_blocks, int32_t max_members, int32_t max_shared_tokens,
                           uint32_t* flags);
int32_t pa_validate_query_starts(const int32_t* q_starts, const int32_t* seq_lens, int32_t B,
                                 int32_t total_q, int32_t max_q, uint32_t* flags);
int32_t pa_validate_append(const int32_t* slot_mapping, const int32_t* block_tables,
                           const int32_t* seq_lens, int32_t B, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks, uint32_t* flags);

/* ------------------------------------------------------------------ read-ceiling aid */

/*
 * pa_read_tiles -- a measurement aid, not part of the attention path: the HBM read rate
 * the decode kernel could reach on its own access pattern. It reads n_tiles tiles of
 * tile_bytes from K and the same bytes from V, tile i at byte offset tile_offsets[i] of
 * both caches, in the order given, the way the stream decode kernel reads its 16-token
 * groups (one wavefront per SIMD, equal contiguous slices of the list, non-temporal
 * 16-byte loads), and does no arithmetic but an XOR of every loaded 32-bit word into one
 * value per wavefront.
 *
 *   k_cache, v_cache  device, 16-byte aligned, cache_bytes each
 *   tile_offsets      device int64 [n_tiles]; each a multiple of 16 with
 *                     offset + tile_bytes <= cache_bytes; the kernel clamps an offset
 *                     outside [0, cache_bytes - tile_bytes] into it and rounds it down to
 *                     16 bytes, so no load leaves the caches
 *   tile_bytes        1024, 2048, 4096, 8192 or 16384 (a 16-token group of one KV head:
 *                     16 x D x element bytes)
 *   sink              device uint32 [4096]; entry w receives the XOR of the words read by
 *                     wavefront w (entries past the device's resident wavefronts are left
 *                     as they are), so the XOR of all entries is the XOR of every word of
 *                     the listed tiles of both caches
 * n_tiles == 0 launches nothing. Asynchronous on `stream`.
 */
int32_t pa_read_tiles(const void* k_cache, const void* v_cache, size_t cache_bytes,
                      const int64_t* tile_offsets, int32_t n_tiles, int32_t tile_bytes,
                      uint32_t* sink, void* stream);

/* ------------------------------------------------------------------ status */

const char* pa_status_string(int32_t status);
/* message of the last failed call on this thread ("" if none) */
const char* pa_last_error(void);
int32_t pa_abi_version(void);

/* ------------------------------------------------------------------ host block allocator */

/*
 * A refcounted allocator of physical block ids that builds block tables on the host
 * ([P2] section 4 "Tiny example": free stack, Allocate, Free, Fork, AppendToken,
 * PhysicalIndex; [P2] section 5 "Copy-on-write sharing"; [P4] sections 3-4). Host memory
 * only; an allocator object is not thread-safe. Every failing call leaves it unchanged.
 *
 * The free list is a stack; initial_free_order (nullable, num_blocks distinct ids) lists
 * it bottom to top, default num_blocks-1 ... 0, so the first allocation of n blocks
 * returns ids n-1 ... 0 in that order.
 */
typedef struct pa_allocator pa_allocator;

pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order);
void pa_alloc_destroy(pa_allocator* a);
/* all-or-nothing: n blocks from the top of the stack, refcount 1 each, into out[n];
 * PA_ERR_NO_BLOCKS ("out of KV blocks: need n, have m") if fewer are free */
int32_t pa_alloc_allocate(pa_allocator* a, int32_t n, int32_t* out);
/* refcount - 1 for each listed block; a block whose count reaches 0 is pushed on the
 * stack; a block freed more often than it is referenced -> PA_ERR_INVALID_ARG */
int32_t pa_alloc_free(pa_allocator* a, const int32_t* blocks, int32_t n);
/* refcount + 1 for each listed (allocated) block; out[n] receives the same ids (the new
 * sequence's table); out may equal blocks */
int32_t pa_alloc_fork(pa_allocator* a, const int32_t* blocks, int32_t n, int32_t* out);
/*
 * Append one token to a sequence whose table is table[0 .. *n_table) (capacity table_cap)
 * and whose length is *seq_len. With pos = *seq_len and j = pos / block_size:
 *   j == *n_table: a fresh block is allocated and appended;
 *   j <  *n_table and table[j] is shared (refcount > 1): a fresh block replaces it, the
 *                 old block's count drops by one, and when pos % block_size != 0 the pair
 *                 (old, fresh) is returned as the copy to make before writing;
 *   otherwise the token goes into table[j] in place.
 * *out_slot = table[j] * block_size + pos % block_size; *seq_len += 1. *out_cow_src and
 * *out_cow_dst are -1 when no copy is needed.
 */
int32_t pa_alloc_append_token(pa_allocator* a, int32_t* table, int32_t* n_table,
                              int32_t table_cap, int32_t* seq_len, int32_t* out_slot,
                              int32_t* out_cow_src, int32_t* out_cow_dst);
/* current refcount of a block (0 if free), or PA_ERR_INVALID_ARG for an id out of range */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block);
int32_t pa_alloc_num_free(const pa_allocator* a);
/* copies the free stack, bottom to top, into out (capacity cap); returns its length */
int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap);
/* tokens per block the allocator was created with */
int32_t pa_alloc_block_size(const pa_allocator* a);

/* ------------------------------------------------------------------ prefix cache */

/*
 * A prefix cache over an allocator ([P2] section 5, "The relationship to prefix
 * caching": hash the token ids of each block, keep a hash -> block map, and let a new
 * sequence whose leading blocks are cached point at them). A block is found by its own
 * tokens and all the tokens before it (the chain from the sequence's first block), and
 * only full blocks are cached. Host memory only, not thread-safe; the allocator must
 * outlive the cache, and the cache holds one reference of its own on every cached block.
 */
typedef struct pa_prefix_cache pa_prefix_cache;

pa_prefix_cache* pa_pcache_create(pa_allocator* a);
/* drops the cache's references (a cached block nobody else holds returns to the free list) */
void pa_pcache_destroy(pa_prefix_cache* c);
/*
 * Table for a new sequence of n_tokens prompt tokens: the longest run of leading full
 * blocks found in the cache is shared (one more reference each), the remaining
 * ceil(n_tokens / block_size) - hits blocks are allocated. When fewer blocks are free
 * than needed, cached blocks no sequence holds are released, least recently used first.
 * *n_table = blocks in table (<= table_cap), *n_cached = tokens whose K/V the shared
 * blocks already hold (hits * block_size). PA_ERR_NO_BLOCKS leaves everything unchanged.
 */
int32_t pa_pcache_acquire(pa_prefix_cache* c, const int32_t* tokens, int32_t n_tokens,
                          int32_t* table, int32_t table_cap, int32_t* n_table,
                          int32_t* n_cached);
/*
 * Make the full blocks of a sequence whose K/V the caller has written findable: block i
 * of table (i < n_tokens / block_size) is cached under tokens[0 .. (i+1) block_size) and
 * gains the cache's reference, unless an equal block is already cached (then that entry
 * is only marked used).
 */
int32_t pa_pcache_publish(pa_prefix_cache* c, const int32_t* tokens, int32_t n_tokens,
                          const int32_t* table, int32_t n_table);
/* release up to n cached blocks no sequence holds, least recently used first; returns
 * how many were released */
int32_t pa_pcache_evict(pa_prefix_cache* c, int32_t n);
int32_t pa_pcache_num_entries(const pa_prefix_cache* c);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
