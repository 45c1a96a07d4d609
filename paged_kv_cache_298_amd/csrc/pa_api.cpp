// pa_api.cpp -- the C ABI declared in include/pa.h: argument validation (pure host code,
// run before any HIP call), launch configuration, workspace sizing and status reporting.
// Kernels are enqueued through the launchers in pa_decode.hip and pa_cache.hip.
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;
int32_t g_partition_override = 0;   // 0 = automatic
int32_t g_path = PA_PATH_AUTO;
int32_t g_stream_waves = 0;         // 0 = every wave the device holds at once
int32_t g_min_slice = pa_internal::kDefaultMinSlice;
int32_t g_longest_first = 1;

int32_t fail(int32_t status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int32_t ok() {
    g_last_error.clear();
    return PA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }


int32_t elt_bytes(int32_t kv_dtype) { return kv_dtype == PA_BF16 ? 2 : (kv_dtype == PA_F32 ? 4 : 0); }

int32_t partition_tokens(int32_t block_size, int32_t max_blocks) {
    if (g_partition_override > 0) return g_partition_override;
    const int64_t cap = (int64_t)block_size * max_blocks;
    if (cap <= pa_internal::kDefaultPartTokens) {
        // one partition covers every sequence: round the capacity up to 64 tokens
        int64_t p = (cap + 63) / 64 * 64;
        return (int32_t)(p < 64 ? 64 : p);
    }
    return pa_internal::kDefaultPartTokens;
}

int32_t n_parts_for(int32_t block_size, int32_t max_blocks) {
    const int64_t cap = (int64_t)block_size * max_blocks;
    const int32_t P = partition_tokens(block_size, max_blocks);
    const int64_t n = (cap + P - 1) / P;
    return (int32_t)(n < 1 ? 1 : n);
}

size_t workspace_layout(int32_t B, int32_t Hq, int32_t D, int32_t n_parts, size_t* ml_offset) {
    if (n_parts <= 1) {
        *ml_offset = 0;
        return 0;
    }
    const size_t rows = (size_t)B * (size_t)Hq * (size_t)n_parts;
    const size_t o_bytes = rows * (size_t)D * sizeof(float);
    const size_t off = (o_bytes + 255) / 256 * 256;
    *ml_offset = off;
    return off + rows * 2 * sizeof(float);
}

// The stream decomposition serves bf16 caches while the per-sequence prefix fits its LDS
// and the group count of the whole batch fits 31 bits.
bool stream_eligible(int32_t kv_dtype, int32_t B, int32_t Hkv, int32_t block_size, int32_t max_blocks) {
    if (kv_dtype != PA_BF16 || B > pa_internal::kMaxStreamB) return false;
    const int64_t groups = ((int64_t)block_size * max_blocks + 15) / 16;
    return (int64_t)B * Hkv * groups < ((int64_t)1 << 31);
}

// Stream decomposition workspace, each section 256-byte aligned: two partial records per
// wave that gets a slice (outputs [G, D] and (max, sum) pairs [G]), one descriptor per
// launched wave and a 4-int header. G counts the query columns of a row (heads, or heads x
// query tokens in the multi-query mode).
struct StreamWs {
    size_t ml, desc, meta, total;
};

StreamWs stream_workspace(int32_t G, int32_t D, int32_t slices, int32_t launched) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t W2 = 2 * (size_t)slices;
    StreamWs w;
    w.ml = up(W2 * (size_t)G * (size_t)D * sizeof(float));
    w.desc = up(w.ml + W2 * (size_t)G * 2 * sizeof(float));
    w.meta = up(w.desc + (size_t)launched * 4 * sizeof(int32_t));
    w.total = w.meta + 4 * sizeof(int32_t);
    return w;
}

// Waves a stream launch starts (the device's resident waves; kMaxStreamWaves when no
// device can be queried) and, of those, the most that get a slice: no more than the batch
// fills with min_slice groups each (T <= B Hkv ceil(capacity / 16) groups).
StreamWs stream_workspace_for(int32_t B, int32_t Hkv, int32_t G, int32_t D, int32_t block_size,
                              int32_t max_blocks) {
    int32_t nw = 0;
    if (pa_internal::stream_waves(g_stream_waves, &nw) != 0 || nw <= 0) nw = pa_internal::kMaxStreamWaves;
    const int64_t gmax = ((int64_t)block_size * max_blocks + 15) / 16;
    int64_t fill = (int64_t)B * Hkv * gmax / (g_min_slice > 0 ? g_min_slice : 1);
    fill = fill < 1 ? 1 : fill;
    return stream_workspace(G, D, fill < nw ? (int32_t)fill : nw, nw);
}

// Blocks of 8 tokens (a 16-token group spans two blocks) are served by the stream
// decomposition only; 0 = no decomposition applies.
int32_t choose_path(int32_t kv_dtype, int32_t B, int32_t Hkv, int32_t block_size, int32_t max_blocks) {
    const bool ok = stream_eligible(kv_dtype, B, Hkv, block_size, max_blocks);
    if (block_size < 16) return (ok && g_path != PA_PATH_PARTITION) ? pa_internal::kPathStream : 0;
    if (g_path == PA_PATH_PARTITION) return pa_internal::kPathPartition;
    if (g_path == PA_PATH_STREAM) return ok ? pa_internal::kPathStream : 0;
    return ok ? pa_internal::kPathStream : pa_internal::kPathPartition;
}

}  // namespace

namespace pa_internal {

MultiPlan multi_plan(int32_t B, int32_t max_q, int32_t Hq, int32_t Hkv, int32_t capacity) {
    MultiPlan m;
    const int64_t rows = (int64_t)max_q * (Hq / Hkv);
    m.nset = rows > 32 && PA_MULTI_MAX_NSET >= 4 ? 4 : (rows > 16 ? 2 : 1);
    m.n_tiles = (int32_t)std::max<int64_t>(1, (rows + 16 * m.nset - 1) / (16 * m.nset));
    int64_t P = std::max<int64_t>(16, ((int64_t)capacity + 15) / 16 * 16);
    const int64_t units = (int64_t)B * Hkv * m.n_tiles;
    while (P > kMultiMinPart && units * ((capacity + P - 1) / P) < kMultiMinWaves)
        P = std::max<int64_t>(kMultiMinPart, (P / 2 + 15) / 16 * 16);
    m.part_tokens = (int32_t)P;
    m.n_parts = (int32_t)std::max<int64_t>(1, (capacity + P - 1) / P);
    return m;
}

}  // namespace pa_internal

namespace {

struct MultiWs {
    pa_internal::MultiPlan plan;
    size_t ml, total;        // the query-tile split's records (0: no split)
    int32_t stream_g;        // > 0: query columns of the stream decomposition, if it applies
    StreamWs sws;
};

// The stream decomposition serves batches whose queries fit one 16-column score tile per
// (sequence, KV head), max_q x G <= 16, with stream_g = 4, 8 or 16 columns.
int32_t multi_stream_g(int32_t B, int32_t max_q, int32_t Hq, int32_t Hkv, int32_t block_size,
                       int32_t max_blocks) {
    const int64_t cols = (int64_t)max_q * (Hq / Hkv);
    if (cols > 16 || !stream_eligible(PA_BF16, B, Hkv, block_size, max_blocks)) return 0;
    return cols <= 4 ? 4 : (cols <= 8 ? 8 : 16);
}

MultiWs multi_workspace(int32_t B, int32_t total_q, int32_t max_q, int32_t Hq, int32_t Hkv,
                        int32_t D, int32_t block_size, int32_t max_blocks) {
    MultiWs w;
    w.plan = pa_internal::multi_plan(B, max_q, Hq, Hkv, block_size * max_blocks);
    w.ml = w.total = 0;
    if (w.plan.n_parts > 1) {
        const size_t rows = (size_t)total_q * (size_t)Hq * (size_t)w.plan.n_parts;
        w.ml = (rows * (size_t)D * sizeof(float) + 255) / 256 * 256;
        w.total = w.ml + rows * 2 * sizeof(float);
    }
    w.stream_g = multi_stream_g(B, max_q, Hq, Hkv, block_size, max_blocks);
    w.sws = stream_workspace_for(B, Hkv, w.stream_g > 0 ? w.stream_g : 4, D, block_size, max_blocks);
    // enough for either decomposition, so the size does not depend on the path setting
    if (w.stream_g > 0 && w.sws.total > w.total) w.total = w.sws.total;
    return w;
}

}  // namespace

namespace {

struct SharedWs {
    int32_t n_pre, n_suf, n_slots, P;
    size_t ml, total;
};

SharedWs shared_workspace(int32_t B, int32_t Hq, int32_t D, int32_t block_size, int32_t max_blocks,
                          int32_t max_shared_tokens) {
    SharedWs w;
    w.P = partition_tokens(block_size, max_blocks);
    const int64_t cap = (int64_t)block_size * max_blocks;
    w.n_pre = (int32_t)(((int64_t)max_shared_tokens + pa_internal::kPrefixTokens - 1) / pa_internal::kPrefixTokens);
    w.n_suf = (int32_t)((cap + w.P - 1) / w.P);
    w.n_slots = w.n_pre + w.n_suf;
    const size_t rows = (size_t)B * (size_t)Hq * (size_t)w.n_slots;
    w.ml = (rows * (size_t)D * sizeof(float) + 255) / 256 * 256;
    w.total = w.ml + rows * 2 * sizeof(float);
    return w;
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        default: return "PA_ERR_UNKNOWN";
    }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

int32_t pa_set_partition_tokens(int32_t tokens) {
    if (tokens != 0 && (tokens < 64 || tokens > pa_internal::kMaxPartTokens || tokens % 64 != 0))
        return fail(PA_ERR_INVALID_ARG, "partition tokens must be 0 or a multiple of 64 in [64, %d], got %d",
                    pa_internal::kMaxPartTokens, tokens);
    g_partition_override = tokens;
    return ok();
}

int32_t pa_decode_partition_tokens(int32_t block_size, int32_t max_blocks) {
    return partition_tokens(block_size, max_blocks);
}

int32_t pa_set_decode_path(int32_t path) {
    if (path != PA_PATH_AUTO && path != PA_PATH_PARTITION && path != PA_PATH_STREAM)
        return fail(PA_ERR_INVALID_ARG, "decode path must be PA_PATH_AUTO, PA_PATH_PARTITION or PA_PATH_STREAM, got %d", path);
    g_path = path;
    return ok();
}

int32_t pa_set_stream_waves(int32_t waves, int32_t min_slice) {
    if (waves < 0 || waves > pa_internal::kMaxStreamWaves || min_slice < 0 || min_slice > (1 << 20))
        return fail(PA_ERR_INVALID_ARG, "stream waves must lie in [0, %d] and min_slice in [0, 2^20], got %d, %d",
                    pa_internal::kMaxStreamWaves, waves, min_slice);
    g_stream_waves = waves;
    g_min_slice = min_slice == 0 ? pa_internal::kDefaultMinSlice : min_slice;
    return ok();
}

int32_t pa_set_multi_order(int32_t longest_first) {
    if (longest_first != 0 && longest_first != 1)
        return fail(PA_ERR_INVALID_ARG, "multi order must be 0 (grid order) or 1 (longest first), got %d",
                    longest_first);
    g_longest_first = longest_first;
    return ok();
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                 int32_t max_blocks, int32_t kv_dtype) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || block_size <= 0 || max_blocks <= 0)
        return 0;
    // the decomposition pa_decode picks for these sizes under the current path setting
    const int32_t path = choose_path(kv_dtype, B, Hkv, block_size, max_blocks);
    if (path == pa_internal::kPathStream)
        return stream_workspace_for(B, Hkv, Hq / Hkv, D, block_size, max_blocks).total;
    if (path != pa_internal::kPathPartition) return 0;
    size_t ml;
    return workspace_layout(B, Hq, D, n_parts_for(block_size, max_blocks), &ml);
}

// pa_decode, and pa_decode_append when nkey != nullptr (the newest token's rows nkey /
// nval [B, Hkv, D] and slots nslots [B] are written to the cache by the same launch on the
// stream decomposition, or by the cache-write kernel just before it otherwise).
static int32_t decode_entry(float* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks, float scale, int32_t kv_dtype, void* workspace,
                            size_t workspace_bytes, void* stream, const void* nkey, const void* nval,
                            const int32_t* nslots) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0 ||
        max_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode: bad sizes B=%d Hq=%d Hkv=%d D=%d block_size=%d num_blocks=%d max_blocks=%d",
                    B, Hq, Hkv, D, block_size, num_blocks, max_blocks);
    if (Hq % Hkv != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (elt_bytes(kv_dtype) == 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: kv_dtype %d is neither PA_F32 nor PA_BF16", kv_dtype);
    if ((int64_t)block_size * max_blocks > (int64_t)1 << 30)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: max_blocks * block_size exceeds 2^30");
    if (B > 65535)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: B=%d exceeds 65535", B);
    const int32_t G = Hq / Hkv;
    if (D != 64 && D != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d not built (64, 128)", D);
    if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d not built (8, 16, 32, 64, 128)", block_size);
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: %d query heads per KV head not built (1, 2, 4, 8)", G);
    if (Hkv > 65535)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: Hkv=%d exceeds 65535", Hkv);
    if (B == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: null pointer argument");
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(seq_lens, 4))
        return fail(PA_ERR_INVALID_ARG, "pa_decode: misaligned pointer (q/out/caches need 16 bytes)");
    if ((int64_t)num_blocks * Hkv * block_size * D * elt_bytes(kv_dtype) < 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: cache size overflows");
    const int32_t path = choose_path(kv_dtype, B, Hkv, block_size, max_blocks);
    if (path == 0)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: the stream decomposition (the only one for "
                    "block_size 8) needs bf16 caches, B <= %d and fewer than 2^31 token groups",
                    pa_internal::kMaxStreamB);
    const int32_t P = partition_tokens(block_size, max_blocks);
    if (path == pa_internal::kPathPartition && P % block_size != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: partition %d not a multiple of block_size %d", P, block_size);
    const int32_t n_parts = n_parts_for(block_size, max_blocks);
    size_t ml_off = 0;
    const StreamWs sws = stream_workspace_for(B, Hkv, G, D, block_size, max_blocks);
    const size_t need = path == pa_internal::kPathStream ? sws.total
                                                         : workspace_layout(B, Hq, D, n_parts, &ml_off);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(PA_ERR_INVALID_ARG, "pa_decode: workspace of %zu bytes needed, %zu given",
                        need, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256))
            return fail(PA_ERR_INVALID_ARG, "pa_decode: workspace must be 256-byte aligned");
    }
    if (path == pa_internal::kPathPartition &&
        ((int64_t)n_parts * Hkv * B > 0x7fffffff || (int64_t)Hq * B > 0x7fffffff))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: %lld work items (or %lld merged rows) exceed the grid limit",
                    (long long)n_parts * Hkv * B, (long long)Hq * B);

    if (pa_internal::validation_on()) {
        const int32_t st = pa_internal::validate_decode_device("pa_decode", block_tables, seq_lens, B, block_size,
                                                               num_blocks, max_blocks, stream);
        if (st != PA_OK) return st;
    }

    pa_internal::DecodeLaunch a;
    a.out = out;
    char* ws = static_cast<char*>(workspace);
    const bool strm = path == pa_internal::kPathStream;
    a.nkey = strm ? nkey : nullptr;
    a.nval = strm ? nval : nullptr;
    a.nslots = strm ? nslots : nullptr;
    if (nkey && !strm) {   // the cache write as its own kernel, then the decode
        const char* err = "";
        const int e = pa_internal::launch_reshape_and_cache(const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                                                            nkey, nval, nslots, B, Hkv, D * elt_bytes(kv_dtype),
                                                            block_size, num_blocks, stream, &err);
        if (e != 0) return fail(PA_ERR_HIP, "pa_decode: cache-write launch failed: %s (%d)", err, e);
    }
    a.ws_o = (!strm && need) ? reinterpret_cast<float*>(ws) : nullptr;
    a.ws_ml = (!strm && need) ? reinterpret_cast<float*>(ws + ml_off) : nullptr;
    a.path = path;
    a.rec_o = strm ? reinterpret_cast<float*>(ws) : nullptr;
    a.rec_ml = strm ? reinterpret_cast<float*>(ws + sws.ml) : nullptr;
    a.desc = strm ? reinterpret_cast<int32_t*>(ws + sws.desc) : nullptr;
    a.meta = strm ? reinterpret_cast<int32_t*>(ws + sws.meta) : nullptr;
    a.stream_waves = g_stream_waves;
    a.min_slice = g_min_slice;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.part_tokens = P;
    a.n_parts = n_parts;
    a.kv_dtype = kv_dtype;
    a.scale = scale;
    a.stream = stream;
    const char* err = "";
    const int e = pa_internal::launch_decode(a, &err);
    if (e != 0) return fail(PA_ERR_HIP, "pa_decode: launch failed: %s (%d)", err, e);
    return ok();
}


int32_t pa_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                  int32_t max_blocks, float scale, int32_t kv_dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
    return decode_entry(out, q, k_cache, v_cache, block_tables, seq_lens, B, Hq, Hkv, D, block_size,
                        num_blocks, max_blocks, scale, kv_dtype, workspace, workspace_bytes, stream,
                        nullptr, nullptr, nullptr);
}

int32_t pa_decode_append(float* out, const void* q, void* k_cache, void* v_cache, const void* key,
                         const void* value, const int32_t* slot_mapping, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks, float scale,
                         int32_t kv_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (B > 0 && (!key || !value || !slot_mapping))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_append: null pointer argument");
    if (B > 0 && (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 4)))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_append: misaligned key, value or slot_mapping");
    if (B > 0 && (int64_t)num_blocks * block_size > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_append: more than 2^31 slots");
    if (B > 0 && pa_internal::validation_on() && elt_bytes(kv_dtype) != 0 && block_size > 0 && num_blocks > 0 &&
        max_blocks > 0) {
        const int32_t st = pa_internal::validate_append_device(slot_mapping, block_tables, seq_lens, B, block_size,
                                                               num_blocks, max_blocks, stream);
        if (st != PA_OK) return st;
    }
    const int32_t st = decode_entry(out, q, k_cache, v_cache, block_tables, seq_lens, B, Hq, Hkv, D, block_size,
                                    num_blocks, max_blocks, scale, kv_dtype, workspace, workspace_bytes, stream,
                                    B > 0 ? key : nullptr, value, slot_mapping);
    if (st != PA_OK) {
        const std::string msg = g_last_error;
        return fail(st, "pa_decode_append -> %s", msg.c_str());
    }
    return ok();
}

int32_t pa_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks, float scale, int32_t kv_dtype, void* stream) {
    // the scratch pa_decode would need for these sizes (0: none, or sizes it rejects)
    const size_t need = pa_decode_workspace_bytes(B, Hq, Hkv, D, block_size, max_blocks, kv_dtype);
    if (need > pa_internal::kScratchBytes)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode_noalloc: these sizes need %zu bytes of scratch; the library holds %zu per "
                    "device (use pa_decode with a workspace)", need, pa_internal::kScratchBytes);
    void* scratch = nullptr;
    if (need > 0) {
        const char* err = "";
        const int e = pa_internal::scratch_pointer(&scratch, &err);
        if (e != 0) return fail(PA_ERR_HIP, "pa_decode_noalloc: scratch address: %s (%d)", err, e);
    }
    const int32_t st = pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, B, Hq, Hkv, D, block_size,
                                 num_blocks, max_blocks, scale, kv_dtype, scratch,
                                 need > 0 ? pa_internal::kScratchBytes : 0, stream);
    if (st != PA_OK) {
        const std::string msg = g_last_error;
        return fail(st, "pa_decode_noalloc -> %s", msg.c_str());
    }
    return ok();
}

size_t pa_decode_shared_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t block_size,
                                        int32_t max_blocks, int32_t max_shared_tokens) {
    if (B <= 0 || Hq <= 0 || D <= 0 || block_size <= 0 || max_blocks <= 0 || max_shared_tokens < 0)
        return 0;
    return shared_workspace(B, Hq, D, block_size, max_blocks, max_shared_tokens).total;
}

int32_t pa_decode_shared(float* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* groups, int32_t n_groups, int32_t max_members,
                         int32_t max_shared_tokens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks, float scale,
                         int32_t kv_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0 ||
        max_blocks <= 0 || n_groups < 0 || max_shared_tokens < 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode_shared: bad sizes B=%d Hq=%d Hkv=%d D=%d block_size=%d num_blocks=%d "
                    "max_blocks=%d n_groups=%d max_shared_tokens=%d",
                    B, Hq, Hkv, D, block_size, num_blocks, max_blocks, n_groups, max_shared_tokens);
    if (Hq % Hkv != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (elt_bytes(kv_dtype) == 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: kv_dtype %d is neither PA_F32 nor PA_BF16", kv_dtype);
    if (kv_dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: only bf16 caches are built");
    if ((int64_t)block_size * max_blocks > (int64_t)1 << 30)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: max_blocks * block_size exceeds 2^30");
    if (max_shared_tokens > block_size * max_blocks)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: max_shared_tokens %d exceeds the table capacity",
                    max_shared_tokens);
    if (B > 65535 || Hkv > 65535)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: B=%d or Hkv=%d exceeds 65535", B, Hkv);
    const int32_t G = Hq / Hkv;
    if (D != 64 && D != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: head_dim %d not built (64, 128)", D);
    if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: block_size %d not built (16, 32, 64, 128)", block_size);
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: %d query heads per KV head not built (1, 2, 4, 8)", G);
    if (n_groups > 0 && (max_members < 1 || (int64_t)max_members * G > pa_internal::kMaxSharedRows))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: max_members %d x %d query heads per KV head "
                    "must lie in [1, %d]", max_members, G, pa_internal::kMaxSharedRows);
    if (B == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || (n_groups > 0 && !groups))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: null pointer argument");
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(seq_lens, 4) || (groups && !aligned(groups, 4)))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: misaligned pointer");
    const SharedWs sw = shared_workspace(B, Hq, D, block_size, max_blocks, max_shared_tokens);
    if (sw.P % block_size != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: partition %d not a multiple of block_size %d", sw.P, block_size);
    if (!workspace || workspace_bytes < sw.total)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: workspace of %zu bytes needed, %zu given",
                    sw.total, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_shared: workspace must be 256-byte aligned");
    // one launch of four items per block: the prefix items, then the suffix partitions
    const int64_t pre_items = (int64_t)n_groups * Hkv * sw.n_pre, suf_items = (int64_t)sw.n_suf * Hkv * B;
    if (pre_items > 0x7fffffff || suf_items > 0x7fffffff || (pre_items + 3) / 4 + (suf_items + 3) / 4 > 0x7fffffff ||
        (int64_t)B * Hq > 0x7fffffff)   // the merge takes one wave per (sequence, query head)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: work items exceed the grid limit");

    if (pa_internal::validation_on()) {
        const int32_t st = pa_internal::validate_shared_device(block_tables, seq_lens, groups, n_groups, B,
                                                               block_size, num_blocks, max_blocks,
                                                               max_members, max_shared_tokens, stream);
        if (st != PA_OK) return st;
    }

    pa_internal::SharedLaunch a;
    a.out = out;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + sw.ml);
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.groups = n_groups > 0 ? groups : nullptr;
    a.n_groups = n_groups;
    a.max_members = n_groups > 0 ? max_members : 1;
    a.max_shared = max_shared_tokens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.pre_tokens = pa_internal::kPrefixTokens;
    a.part_tokens = sw.P;
    a.n_pre = n_groups > 0 ? sw.n_pre : 0;
    a.n_suf = sw.n_suf;
    a.n_slots = sw.n_slots;
    a.scale = scale;
    a.stream = stream;
    const char* err = "";
    const int e = pa_internal::launch_decode_shared(a, &err);
    if (e != 0) return fail(PA_ERR_HIP, "pa_decode_shared: launch failed: %s (%d)", err, e);
    return ok();
}



size_t pa_decode_multi_workspace_bytes(int32_t B, int32_t total_q, int32_t max_q, int32_t Hq,
                                       int32_t Hkv, int32_t D, int32_t block_size,
                                       int32_t max_blocks) {
    if (B <= 0 || total_q <= 0 || max_q <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 ||
        block_size <= 0 || max_blocks <= 0 || (int64_t)block_size * max_blocks > (int64_t)1 << 30)
        return 0;
    return multi_workspace(B, total_q, max_q, Hq, Hkv, D, block_size, max_blocks).total;
}

int32_t pa_decode_multi(float* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* q_starts, int32_t B, int32_t total_q, int32_t max_q,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks, float scale, int32_t kv_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (B < 0 || total_q < 0 || max_q < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 ||
        num_blocks <= 0 || max_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode_multi: bad sizes B=%d total_q=%d max_q=%d Hq=%d Hkv=%d D=%d "
                    "block_size=%d num_blocks=%d max_blocks=%d",
                    B, total_q, max_q, Hq, Hkv, D, block_size, num_blocks, max_blocks);
    if (Hq % Hkv != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (elt_bytes(kv_dtype) == 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: kv_dtype %d is neither PA_F32 nor PA_BF16", kv_dtype);
    if (kv_dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_multi: only bf16 caches are built");
    if ((int64_t)block_size * max_blocks > (int64_t)1 << 30)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: max_blocks * block_size exceeds 2^30");
    if (total_q > 0 && max_q == 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: max_q is 0 with %d queries", total_q);
    // query rows per sequence (max_q x G) and rows in all (total_q x Hq) are int on the device
    if ((int64_t)max_q * (Hq / Hkv) > ((int64_t)1 << 30) || (int64_t)total_q * Hq > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_multi: %d queries x %d heads exceed the row range",
                    total_q, Hq);
    if (D != 64 && D != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_multi: head_dim %d not built (64, 128)", D);
    if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_multi: block_size %d not built (16, 32, 64, 128)", block_size);
    if (B == 0 || total_q == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !q_starts)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: null pointer argument");
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(q_starts, 4))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: misaligned pointer");
    const MultiWs mw = multi_workspace(B, total_q, max_q, Hq, Hkv, D, block_size, max_blocks);
    const pa_internal::MultiPlan& pl = mw.plan;
    const int32_t stream_g = g_path == PA_PATH_PARTITION ? 0 : mw.stream_g;
    const int64_t items = (int64_t)Hkv * pl.n_tiles * pl.n_parts * B;
    if (items > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_multi: work items exceed the grid limit");
    if (stream_g == 0 && pl.n_parts > 1 && (total_q > 65535 || Hq > 65535))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_multi: %d queries of a split launch exceed 65535", total_q);
    if (mw.total > 0) {
        if (!workspace || workspace_bytes < mw.total)
            return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: workspace of %zu bytes needed, %zu given",
                        mw.total, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256))
            return fail(PA_ERR_INVALID_ARG, "pa_decode_multi: workspace must be 256-byte aligned");
    }

    if (pa_internal::validation_on()) {
        const int32_t st = pa_internal::validate_multi_device(block_tables, seq_lens, q_starts, B, total_q, max_q,
                                                              block_size, num_blocks, max_blocks, stream);
        if (st != PA_OK) return st;
    }

    pa_internal::MultiLaunch a;
    a.out = out;
    a.ws_o = mw.total > 0 ? static_cast<float*>(workspace) : nullptr;
    a.ws_ml = mw.total > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + mw.ml) : nullptr;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.q_starts = q_starts;
    a.B = B;
    a.total_q = total_q;
    a.max_q = max_q;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.nset = pl.nset;
    a.n_tiles = pl.n_tiles;
    a.part_tokens = pl.part_tokens;
    a.n_parts = pl.n_parts;
    a.longest_first = g_longest_first;
    a.stream_g = stream_g;
    a.rec_o = nullptr;
    a.rec_ml = nullptr;
    a.desc = nullptr;
    a.meta = nullptr;
    if (stream_g > 0) {
        char* ws = static_cast<char*>(workspace);
        a.rec_o = reinterpret_cast<float*>(ws);
        a.rec_ml = reinterpret_cast<float*>(ws + mw.sws.ml);
        a.desc = reinterpret_cast<int32_t*>(ws + mw.sws.desc);
        a.meta = reinterpret_cast<int32_t*>(ws + mw.sws.meta);
    }
    a.stream_waves = g_stream_waves;
    a.min_slice = g_min_slice;
    a.scale = scale;
    a.stream = stream;
    const char* err = "";
    const int e = pa_internal::launch_decode_multi(a, &err);
    if (e != 0) return fail(PA_ERR_HIP, "pa_decode_multi: launch failed: %s (%d)", err, e);
    return ok();
}

int32_t pa_reshape_and_cache(void* k_cache, void* v_cache, const void* key, const void* value,
                             const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                             int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                             void* stream) {
    const int32_t eb = elt_bytes(kv_dtype);
    if (eb == 0)
        return fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: kv_dtype %d is neither PA_F32 nor PA_BF16", kv_dtype);
    if (T < 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: bad sizes T=%d Hkv=%d D=%d block_size=%d num_blocks=%d",
                    T, Hkv, D, block_size, num_blocks);
    if (D > 512 || (D * eb) % 16 != 0)
        return fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: head_dim %d (rows must be whole 16-byte units, <= 512)", D);
    if ((int64_t)num_blocks * block_size > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: more than 2^31 slots");
    if (T == 0) return ok();
    if (!k_cache || !v_cache || !key || !value || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: null pointer argument");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(key, 16) || !aligned(value, 16) ||
        !aligned(slot_mapping, 4))
        return fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: misaligned pointer");
    if (pa_internal::validation_on()) {
        const int32_t st = pa_internal::validate_slots_device(slot_mapping, T, block_size, num_blocks, stream);
        if (st != PA_OK) return st;
    }
    const char* err = "";
    const int e = pa_internal::launch_reshape_and_cache(k_cache, v_cache, key, value, slot_mapping,
                                                        T, Hkv, D * eb, block_size, num_blocks,
                                                        stream, &err);
    if (e != 0) return fail(PA_ERR_HIP, "pa_reshape_and_cache: launch failed: %s (%d)", err, e);
    return ok();
}

int32_t pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t N,
                       int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                       int32_t kv_dtype, void* stream) {
    const int32_t eb = elt_bytes(kv_dtype);
    if (eb == 0)
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: kv_dtype %d is neither PA_F32 nor PA_BF16", kv_dtype);
    if (N < 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: bad sizes N=%d Hkv=%d D=%d block_size=%d num_blocks=%d",
                    N, Hkv, D, block_size, num_blocks);
    const int64_t block_bytes = (int64_t)Hkv * block_size * D * eb;
    if (block_bytes % 16 != 0)
        return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: block of %lld bytes is not a whole number of 16-byte units",
                    (long long)block_bytes);
    if (N == 0) return ok();
    if (!k_cache || !v_cache || !block_pairs)
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: null pointer argument");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 4))
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: misaligned pointer");
    if (pa_internal::validation_on()) {
        const int32_t st = pa_internal::validate_pairs_device(block_pairs, N, num_blocks, stream);
        if (st != PA_OK) return st;
    }
    const char* err = "";
    const int e = pa_internal::launch_copy_blocks(k_cache, v_cache, block_pairs, N, block_bytes,
                                                  num_blocks, stream, &err);
    if (e != 0) return fail(PA_ERR_HIP, "pa_copy_blocks: launch failed: %s (%d)", err, e);
    return ok();
}

int32_t pa_read_tiles(const void* k_cache, const void* v_cache, size_t cache_bytes,
                      const int64_t* tile_offsets, int32_t n_tiles, int32_t tile_bytes,
                      uint32_t* sink, void* stream) {
    if (n_tiles < 0 || (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 &&
                        tile_bytes != 8192 && tile_bytes != 16384))
        return fail(PA_ERR_INVALID_ARG, "pa_read_tiles: bad sizes n_tiles=%d tile_bytes=%d (1024..16384, a power of 2)",
                    n_tiles, tile_bytes);
    if (n_tiles == 0) return ok();
    if (!k_cache || !v_cache || !tile_offsets || !sink)
        return fail(PA_ERR_INVALID_ARG, "pa_read_tiles: null pointer argument");
    if (cache_bytes < (size_t)tile_bytes)
        return fail(PA_ERR_INVALID_ARG, "pa_read_tiles: caches of %zu bytes hold no tile of %d bytes",
                    cache_bytes, tile_bytes);
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(tile_offsets, 8) || !aligned(sink, 4))
        return fail(PA_ERR_INVALID_ARG, "pa_read_tiles: misaligned pointer");
    const char* err = "";
    const int e = pa_internal::launch_read_tiles(k_cache, v_cache, cache_bytes, tile_offsets, n_tiles, tile_bytes,
                                                 sink, stream, &err);
    if (e != 0) return fail(PA_ERR_HIP, "pa_read_tiles: launch failed: %s (%d)", err, e);
    return ok();
}

}  // extern "C"

namespace pa_internal {
// The allocator entry points (allocator.cpp) report through the same thread-local message.
int32_t set_error(int32_t status, const char* msg) { return fail(status, "%s", msg); }
int32_t clear_error() { return ok(); }
}  // namespace pa_internal
