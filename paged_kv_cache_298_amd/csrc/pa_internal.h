// pa_internal.h -- declarations shared by the C-ABI layer (plain C++) and the HIP kernel
// launchers. No HIP types appear here, so the ABI layer builds with any C++ compiler.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa_internal {

// Everything one pa_decode call needs, already validated on the host.
struct DecodeLaunch {
    float* out;              // [B, Hq, D]
    float* ws_o;             // [B, Hq, n_parts, D]  (unused when n_parts == 1)
    float* ws_ml;            // [B, Hq, n_parts, 2]  (running max in log2 units, sum)
    const void* q;           // [B, Hq, D]
    const void* k;           // [num_blocks, Hkv, bs, D]
    const void* v;
    const int32_t* tables;   // [B, max_blocks]
    const int32_t* lens;     // [B]
    int32_t B, Hq, Hkv, D, bs, num_blocks, max_blocks;
    int32_t part_tokens;     // tokens per partition (multiple of 64, <= kMaxPartTokens)
    int32_t n_parts;         // ceil(max_blocks * bs / part_tokens)
    int32_t kv_dtype;        // PA_F32 / PA_BF16
    float scale;
    void* stream;
    // stream decomposition (path == kPathStream)
    int32_t path;            // kPathPartition or kPathStream
    float* rec_o;            // [2 * slices, G, D]
    float* rec_ml;           // [2 * slices, G, 2]
    int32_t* desc;           // [launched waves, 4]
    int32_t* meta;           // [4]
    int32_t stream_waves;    // 0 = every wave the device holds at once
    int32_t min_slice;       // fewest 16-token groups per wave
    // pa_decode_append on the stream decomposition: the newest token's K and V rows
    // [B, Hkv, D] and slots [B], written by the decode launch itself (nkey == nullptr: none)
    const void* nkey;
    const void* nval;
    const int32_t* nslots;
};

constexpr int kMaxPartTokens = 1024;
constexpr int kDefaultPartTokens = 512;
constexpr int kPathPartition = 1;
constexpr int kPathStream = 2;
constexpr int kMaxStreamB = 4096;        // sequences whose prefix fits the kernel's LDS
constexpr int kMaxStreamWaves = 4096;    // resident waves the records are sized for
constexpr int kDefaultMinSlice = 8;

// Shared-prefix decode (pa_decode_shared), already validated on the host.
struct SharedLaunch {
    float* out;
    float* ws_o;             // [B, Hq, n_slots, D]
    float* ws_ml;            // [B, Hq, n_slots, 2]
    const void* q;
    const void* k;
    const void* v;
    const int32_t* tables;
    const int32_t* lens;
    const int32_t* groups;   // device [n_groups, 3]
    int32_t n_groups, max_members, max_shared;
    int32_t B, Hq, Hkv, D, bs, num_blocks, max_blocks;
    int32_t pre_tokens;      // tokens per prefix partition
    int32_t part_tokens;     // tokens per partition of the sequences' own tokens
    int32_t n_pre, n_suf, n_slots;
    float scale;
    void* stream;
};

#ifndef PA_PREFIX_TOKENS
#define PA_PREFIX_TOKENS 256
#endif
constexpr int kPrefixTokens = PA_PREFIX_TOKENS;
constexpr int kMaxSharedRows = 64;      // members x G query rows per KV head

// Multi-query decode with a causal mask (pa_decode_multi), already validated on the host.
struct MultiLaunch {
    float* out;              // [total_q, Hq, D]
    float* ws_o;             // [total_q, Hq, n_parts, D] (n_parts > 1 only)
    float* ws_ml;            // [total_q, Hq, n_parts, 2]
    const void* q;           // [total_q, Hq, D]
    const void* k;
    const void* v;
    const int32_t* tables;
    const int32_t* lens;
    const int32_t* q_starts; // device [B + 1]
    int32_t B, total_q, max_q, Hq, Hkv, D, bs, num_blocks, max_blocks;
    int32_t nset;            // query tile = 16 nset rows
    int32_t n_tiles, part_tokens, n_parts;
    int32_t longest_first;   // query-tile work handed out longest first (else grid order)
    // stream decomposition (stream_g > 0): the decode kernel's slices with stream_g query
    // columns (token x head) per row instead of query tiles
    int32_t stream_g;
    float* rec_o;
    float* rec_ml;
    int32_t* desc;
    int32_t* meta;
    int32_t stream_waves, min_slice;
    float scale;
    void* stream;
};

// How pa_decode_multi splits its work: query tiles of 16 nset rows, token partitions of
// part_tokens (a multiple of 16; one partition when that already gives enough waves).
struct MultiPlan {
    int32_t nset, n_tiles, part_tokens, n_parts;
};
MultiPlan multi_plan(int32_t B, int32_t max_q, int32_t Hq, int32_t Hkv, int32_t capacity);
#ifndef PA_MULTI_MIN_WAVES
#define PA_MULTI_MIN_WAVES 2048
#endif
#ifndef PA_MULTI_MAX_NSET
#define PA_MULTI_MAX_NSET 4
#endif
#ifndef PA_MULTI_MIN_PART
#define PA_MULTI_MIN_PART 256
#endif
constexpr int kMultiMinWaves = PA_MULTI_MIN_WAVES;   // split the tokens until this many items exist
constexpr int kMultiMinPart = PA_MULTI_MIN_PART;     // ... but not below this many tokens per partition

// Waves the stream decomposition launches on the current device: override_waves (> 0,
// rounded up to a multiple of 4), else one per SIMD; at most kMaxStreamWaves. Returns 0, or
// a HIP error code when the device cannot be queried.
int stream_waves(int32_t override_waves, int32_t* nw);

// Scratch of pa_decode_noalloc: a device array of kScratchBytes per GPU held by the
// library (pa_noalloc.hip); scratch_pointer gives its address on the current device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
int scratch_pointer(void** ptr, const char** err);

// Each returns 0 on success or a nonzero HIP error code (message in *err).
int launch_decode(const DecodeLaunch& a, const char** err);
int launch_decode_shared(const SharedLaunch& a, const char** err);
int launch_decode_multi(const MultiLaunch& a, const char** err);
int launch_multi_stream(const MultiLaunch& a, const char** err);   // stream_g > 0
int launch_reshape_and_cache(void* k_cache, void* v_cache, const void* key, const void* value,
                             const int32_t* slot_mapping, int32_t T, int32_t Hkv,
                             int32_t row_bytes, int32_t block_size, int32_t num_blocks,
                             void* stream, const char** err);
int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t N,
                       int64_t block_bytes, int32_t num_blocks, void* stream, const char** err);
int launch_read_tiles(const void* k, const void* v, size_t cache_bytes, const int64_t* offs, int32_t n,
                      int32_t tile_bytes, uint32_t* sink, void* stream, const char** err);

// Debug validation pass (validate.cpp): whether it is on, and the checks each kernel entry
// point runs on host copies of its device index arrays (PA_OK or a status with the message
// set).
bool validation_on();
int32_t validate_decode_device(const char* who, const int32_t* tables, const int32_t* lens, int32_t B,
                               int32_t block_size, int32_t num_blocks, int32_t max_blocks, void* stream);
int32_t validate_shared_device(const int32_t* tables, const int32_t* lens, const int32_t* groups,
                               int32_t n_groups, int32_t B, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks, int32_t max_members, int32_t max_shared_tokens,
                               void* stream);
int32_t validate_multi_device(const int32_t* tables, const int32_t* lens, const int32_t* q_starts,
                              int32_t B, int32_t total_q, int32_t max_q, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks, void* stream);
int32_t validate_slots_device(const int32_t* slots, int32_t T, int32_t block_size, int32_t num_blocks,
                              void* stream);
int32_t validate_pairs_device(const int32_t* pairs, int32_t N, int32_t num_blocks, void* stream);
int32_t validate_append_device(const int32_t* slots, const int32_t* tables, const int32_t* lens, int32_t B,
                               int32_t block_size, int32_t num_blocks, int32_t max_blocks, void* stream);
// bytes from device memory to host memory on `stream`, waiting for the copy (0 or a HIP
// error code, message in *err)
int copy_to_host(void* dst, const void* src, size_t bytes, void* stream, const char** err);

// Thread-local error message of the C ABI (pa_last_error); set_error returns status.
int32_t set_error(int32_t status, const char* msg);
int32_t clear_error();

}  // namespace pa_internal
