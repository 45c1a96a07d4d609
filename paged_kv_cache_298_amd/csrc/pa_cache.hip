// pa_cache.hip -- the two small kernels that feed paged decode attention on gfx950.
//
// reshape_and_cache: write each new token's K and V row of every KV head to its physical
//   slot s, i.e. block s / block_size, offset s % block_size. The slot is the flat index
//   of [P2] "Paged Attention" tutorial (infra.pidoku.co.in), section 4 "Tiny example",
//   PhysicalIndex: table[pos / block_size] * block_size + pos % block_size.
// copy_blocks: clone whole physical blocks (K and V, all heads and slots) before a write
//   into a shared block, the copy-on-write of [P2] section 5 "Copy-on-write sharing" and
//   [P4] "PagedAttention & KV-Cache Management in High-Throughput LLM Serving"
//   (subroutine-cs.cc), section 3.
// Both are bit copies moved in 16-byte units, one unit per lane per access, consecutive
// lanes on consecutive units, so every wave-wide access is 1 KiB of contiguous bytes.
// read_tiles (pa_read_tiles): a measurement aid, not part of the attention path; it reads
//   a list of K/V tiles the way the stream decode kernel does, with no arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One thread per 16-byte unit of a (token, KV head) row; K and V moved together.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    u32x4_t* __restrict__ kc, u32x4_t* __restrict__ vc, const u32x4_t* __restrict__ key,
    const u32x4_t* __restrict__ value, const int32_t* __restrict__ slots, int64_t total,
    int Hkv, int row_units, int bs, int64_t nslots) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int c = (int)(idx % row_units);
    const int64_t r = idx / row_units;     // token * Hkv + head
    const int g = (int)(r % Hkv);
    const int64_t i = r / Hkv;
    const int s = slots[i];
    if (s < 0 || (int64_t)s >= nslots) return;
    const int64_t blk = s / bs;
    const int64_t off = s % bs;
    const int64_t dst = ((blk * Hkv + g) * bs + off) * row_units + c;
    const u32x4_t kx = key[idx];
    const u32x4_t vx = value[idx];
    kc[dst] = kx;
    vc[dst] = vx;
}

constexpr int kCopyUnitsPerThread = 4;

// blockIdx.y = pair index; each block moves 256 * 4 units (16 KiB) of K and of V.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4_t* __restrict__ kc,
                                                          u32x4_t* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t block_units, int num_blocks) {
    const int n = blockIdx.y;
    const int src = pairs[2 * n];
    const int dst = pairs[2 * n + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const int64_t base = (int64_t)blockIdx.x * (256 * kCopyUnitsPerThread) + threadIdx.x;
    const u32x4_t* ks = kc + (int64_t)src * block_units;
    const u32x4_t* vs = vc + (int64_t)src * block_units;
    u32x4_t* kd = kc + (int64_t)dst * block_units;
    u32x4_t* vd = vc + (int64_t)dst * block_units;
    u32x4_t kx[kCopyUnitsPerThread], vx[kCopyUnitsPerThread];
#pragma unroll
    for (int j = 0; j < kCopyUnitsPerThread; ++j) {
        const int64_t u = base + j * 256;
        if (u < block_units) {
            kx[j] = ks[u];
            vx[j] = vs[u];
        }
    }
#pragma unroll
    for (int j = 0; j < kCopyUnitsPerThread; ++j) {
        const int64_t u = base + j * 256;
        if (u < block_units) {
            kd[u] = kx[j];
            vd[u] = vx[j];
        }
    }
}

// Read-ceiling aid (pa_read_tiles): stream a given list of tiles, each tile_bytes of K at
// a byte offset and the same bytes of V at that offset, the way the stream decode kernel
// reads its 16-token groups -- one wave per SIMD, equal contiguous slices of the list,
// the offsets of 64 tiles at a time held in lanes, non-temporal 16-byte loads -- but with
// no arithmetic: every loaded word is folded by XOR into one value per wave, which keeps
// the loads live and lets the result be checked bit for bit. NCH = tile_bytes / 1024;
// about 32 loads per lane are in flight per batch.
// Offsets are clamped into [0, max_off] and rounded down to 16 bytes (max_off =
// cache_bytes - tile_bytes, itself a multiple of 16), so every load stays inside the caches.
template <int NCH>
__global__ __launch_bounds__(256) void read_tiles_kernel(const char* __restrict__ k,
                                                         const char* __restrict__ v,
                                                         const int64_t* __restrict__ offs, int n,
                                                         int nw, int64_t max_off,
                                                         uint32_t* __restrict__ sink) {
    constexpr int TB = NCH >= 16 ? 1 : 16 / NCH;   // tiles per batch
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (w >= nw) return;
    const int s0 = (int)((int64_t)w * n / nw);
    const int s1 = (int)((int64_t)(w + 1) * n / nw);
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int base = s0; base < s1; base += 64) {
        int idx = base + lane;
        idx = idx < s1 ? idx : s1 - 1;
        int64_t my = offs[idx];
        my = my < 0 ? 0 : (my > max_off ? max_off : my);
        my &= ~(int64_t)15;
        const uint32_t my_lo = (uint32_t)my, my_hi = (uint32_t)((uint64_t)my >> 32);
        const int cnt = min(64, s1 - base);
        for (int u0 = 0; u0 < cnt; u0 += TB) {
            u32x4_t r[TB][2 * NCH];
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                // a batch past the slice's last tile reads the first tile of the caches
                // instead (not XORed; one tile every wave reads stays in cache)
                const int tt = min(u0 + t, cnt - 1);
                const int64_t off = u0 + t < cnt
                    ? (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(my_hi, tt) << 32) |
                                (uint64_t)(uint32_t)__builtin_amdgcn_readlane(my_lo, tt))
                    : 0;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    r[t][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(k + off + i * 1024 + lane * 16));
                    r[t][NCH + i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(v + off + i * 1024 + lane * 16));
                }
            }
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (u0 + t < cnt) {
#pragma unroll
                    for (int i = 0; i < 2 * NCH; ++i) acc ^= r[t][i];
                }
        }
    }
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
    if (lane == 0) sink[w] = x;
}

}  // namespace

namespace pa_internal {

int launch_reshape_and_cache(void* k_cache, void* v_cache, const void* key, const void* value,
                             const int32_t* slot_mapping, int32_t T, int32_t Hkv,
                             int32_t row_bytes, int32_t block_size, int32_t num_blocks,
                             void* stream, const char** err) {
    if (T == 0) return 0;
    const int row_units = row_bytes / 16;
    const int64_t total = (int64_t)T * Hkv * row_units;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<u32x4_t*>(k_cache),
                       static_cast<u32x4_t*>(v_cache), static_cast<const u32x4_t*>(key),
                       static_cast<const u32x4_t*>(value), slot_mapping, total, (int)Hkv,
                       row_units, (int)block_size, (int64_t)num_blocks * block_size);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t N,
                       int64_t block_bytes, int32_t num_blocks, void* stream, const char** err) {
    if (N == 0) return 0;
    const int64_t units = block_bytes / 16;
    const int64_t per_block = 256 * kCopyUnitsPerThread;
    const int64_t gx = (units + per_block - 1) / per_block;
    constexpr int32_t kMaxGridY = 65535;
    for (int32_t first = 0; first < N; first += kMaxGridY) {
        const int32_t n = N - first < kMaxGridY ? N - first : kMaxGridY;
        hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)n), dim3(256), 0,
                           reinterpret_cast<hipStream_t>(stream), static_cast<u32x4_t*>(k_cache),
                           static_cast<u32x4_t*>(v_cache), block_pairs + 2 * (int64_t)first,
                           units, (int)num_blocks);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

int copy_to_host(void* dst, const void* src, size_t bytes, void* stream, const char** err) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

int launch_read_tiles(const void* k, const void* v, size_t cache_bytes, const int64_t* offs, int32_t n,
                      int32_t tile_bytes, uint32_t* sink, void* stream, const char** err) {
    // one 4-wave workgroup per CU, as the stream decode kernel runs: each workgroup
    // reserves just over half of a CU's LDS, so no CU takes two
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int dev = 0, cus = 0, per_cu = 0, per_block = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e == hipSuccess) {
        int nw = cus * 4;
        nw = nw > kMaxStreamWaves ? kMaxStreamWaves : nw;
        size_t lds = (size_t)per_cu / 2 + 1024;
        if (lds > (size_t)per_block) lds = 0;
        const dim3 grid((nw + 3) / 4), block(256);
        const char* kc = static_cast<const char*>(k);
        const char* vc = static_cast<const char*>(v);
        const int64_t mo = (int64_t)((cache_bytes - (size_t)tile_bytes) & ~(size_t)15);
        switch (tile_bytes) {
            case 1024: hipLaunchKernelGGL(read_tiles_kernel<1>, grid, block, lds, st, kc, vc, offs, n, nw, mo, sink); break;
            case 2048: hipLaunchKernelGGL(read_tiles_kernel<2>, grid, block, lds, st, kc, vc, offs, n, nw, mo, sink); break;
            case 4096: hipLaunchKernelGGL(read_tiles_kernel<4>, grid, block, lds, st, kc, vc, offs, n, nw, mo, sink); break;
            case 8192: hipLaunchKernelGGL(read_tiles_kernel<8>, grid, block, lds, st, kc, vc, offs, n, nw, mo, sink); break;
            default: hipLaunchKernelGGL(read_tiles_kernel<16>, grid, block, lds, st, kc, vc, offs, n, nw, mo, sink); break;
        }
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

}  // namespace pa_internal
