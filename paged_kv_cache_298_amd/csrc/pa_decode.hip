// pa_decode.hip -- paged decode attention for gfx950 (MI355X).
//
// Sources: [P1] "PagedAttention" (inferensys.com glossary): the kernel reads the block
// table, gathers K/V from scattered physical blocks, handles a partly filled last block
// and fuses the gather into the attention; [P2] "Paged Attention" tutorial
// (infra.pidoku.co.in), section 5 "The kernel side": grid over (sequence, head), loop over
// ceil(ctx / block_size) blocks, phys = table[blk], q.k and a softmax accumulated per
// block. That page's sketch and its cache layout were written for NVIDIA warps; this
// file keeps what it computes and lays the work out for 64-lane CDNA4 wavefronts.
//
// Work decomposition. One wavefront (one 64-thread workgroup) per
// (partition of P tokens, KV head g, sequence b). All G = Hq / Hkv query heads that read
// KV head g are served by the same wavefront, so every K/V byte is fetched from HBM once.
// Sequences longer than P are split; a second kernel combines the partitions exactly.
//
// Per partition, in three passes over LDS:
//   1. QK^T on the matrix cores. For each 16-token group the K rows (a contiguous
//      16 x D tile of the block) are the A operand of v_mfma_f32_16x16x32_bf16 (fp32 data:
//      v_mfma_f32_16x16x4_f32) and the G query rows, zero-padded to 16, are the B operand.
//      Each lane feeds its A operand straight from one 16-byte global load of its token's
//      row; no LDS staging. Scores (scaled, in log2 units) go to LDS; tokens past the
//      sequence end become -inf by a select, so NaN garbage in unused slots never leaks.
//   2. Per-head partition max (cross-lane), p = exp2(s - m) in place, per-head sum.
//   3. PV on the vector ALUs: each wave-wide 16-byte load covers 1 KiB of contiguous V
//      rows; lanes own 8 (bf16) or 4 (fp32) columns of one row, read that row's G
//      probabilities from LDS by broadcast, and accumulate G x 8 fp32 partial outputs;
//      rows are summed across lanes at the end. V rows past the sequence end are zeroed
//      by a select before use.
// Block-table entries for the partition are prefetched into LDS once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa_internal.h"

// Build-time tuning knobs: ring depth (16-token groups in flight per wave) of the bf16 and
// fp32 kernels, and whether the bf16 kernel computes a ring's groups back to back before
// refilling them.
#ifndef PA_BF16_DEPTH
#define PA_BF16_DEPTH 4
#endif
#ifndef PA_BF16_CHUNK
#define PA_BF16_CHUNK 8
#endif
#ifndef PA_BF16_QLDS
#define PA_BF16_QLDS 0
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 4
#endif

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct Params {
    float* out;
    float* ws_o;
    float2* ws_ml;
    const char* q;
    const char* k;
    const char* v;
    const int32_t* tables;
    const int32_t* lens;
    int B, Hq, Hkv, bs, bs_shift, num_blocks, max_blocks, part_tokens, n_parts;
    float scale_log2;
};

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16 x 16 score tile: rows = the 16 tokens of a group, columns = query heads (G used).
// Lane l holds rows 4*(l/16) + i (i = 0..3) of column l % 16 on return.
template <bool BF16, int KL>
__device__ __forceinline__ f32x4_t qk_tile(const u32x4_t (&kf)[KL], const u32x4_t (&qf)[KL]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < KL; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[c]),
                                                          __builtin_bit_cast(bf16x8_t, qf[c]),
                                                          acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int c = 0; c < KL; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[c][j]),
                                                           __uint_as_float(qf[c][j]), acc, 0, 0,
                                                           0);
    }
    return acc;
}

#ifndef PA_DECODE_NT
#define PA_DECODE_NT 0
#endif

// K/V bytes are read once per call: stream them past the caches when PA_DECODE_NT is set.
__device__ __forceinline__ u32x4_t load16(const u32x4_t* ptr) {
#if PA_DECODE_NT
    return __builtin_nontemporal_load(ptr);
#else
    return *ptr;
#endif
}

// The workgroup is exactly one wavefront, so LDS traffic between its lanes needs only
// ordering, not a workgroup barrier: LDS instructions of one wave execute in issue order.
// Wavefront-scope fences keep the compiler from reordering across this point and, unlike
// a workgroup barrier, do not wait for outstanding global loads.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work item of this workgroup. The grid is one-dimensional and ordered KV head fastest,
// then sequence, then partition. Consecutive workgroups are dealt round-robin to the
// eight XCDs, each of which has its own L2 and its own link to HBM, so this order gives
// every XCD the same mix of heads, sequences and partitions: with 8 KV heads, XCD k serves
// KV head k of every partition, an exact eighth of the bytes. (Partition-fastest order
// would send every sequence's first partition, the one that always exists, to one XCD.)
__device__ __forceinline__ void work_item(const Params& p, int& g, int& b, int& part) {
    const int id = blockIdx.x;
    g = id % p.Hkv;
    const int rest = id / p.Hkv;
    b = rest % p.B;
    part = rest / p.B;
}

template <int G>
__device__ __forceinline__ void load_probs(const float* __restrict__ src, float (&p)[G]) {
    if constexpr (G % 4 == 0) {
#pragma unroll
        for (int h = 0; h < G; h += 4) {
            const float4 x = *reinterpret_cast<const float4*>(src + h);
            p[h] = x.x; p[h + 1] = x.y; p[h + 2] = x.z; p[h + 3] = x.w;
        }
    } else if constexpr (G == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        p[0] = x.x; p[1] = x.y;
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) p[h] = src[h];
    }
}

template <bool BF16, int D, int G, int DEPTH>
__global__ __launch_bounds__(64) void decode_partition_kernel(Params p) {
    constexpr int EB = BF16 ? 2 : 4;   // bytes per element
    constexpr int E = 16 / EB;         // elements per 16-byte load
    constexpr int KQ = D / 4;          // elements of a K row fed by one lane (quarter row)
    constexpr int NL = KQ / E;         // 16-byte loads per lane per 16-token group (K or V)
    constexpr int O = D / E;           // lanes covering one V row
    constexpr int R = 64 / O;          // V rows per wave-wide load
    constexpr int ROW = D * EB;        // bytes per cached row
    static_assert(NL >= 1 && R >= 1 && 16 / R == NL, "unsupported head size");

    extern __shared__ float smem[];
    float* s_lds = smem;                                            // [part_tokens][G]
    int* tbl = reinterpret_cast<int*>(smem + p.part_tokens * G);    // [part_tokens / 16]

    const int lane = threadIdx.x;
    int g, b, part;
    work_item(p, g, b, part);
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int t0 = part * p.part_tokens;
    const int hq0 = g * G;

    if (t0 >= L) {
        if (part == 0) {   // empty sequence: a zero row per head
            for (int i = lane; i < G * D; i += 64)
                p.out[((int64_t)b * p.Hq + hq0) * D + i] = 0.f;
        }
        return;
    }
    const int ntok = min(p.part_tokens, L - t0);
    const int ngroups = (ntok + 15) >> 4;
    const int nparts_b = (L + p.part_tokens - 1) / p.part_tokens;

    // block-table slice of this partition -> LDS (entries clamped into the pool)
    const int blk0 = t0 >> p.bs_shift;
    const int nblk = ((ntok - 1) >> p.bs_shift) + 1;
    const int32_t* trow = p.tables + (int64_t)b * p.max_blocks + blk0;
    for (int i = lane; i < nblk; i += 64) {
        int e = trow[i];
        e = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
        tbl[i] = e;
    }

    // Head-dim split of the QK contraction: MFMA step c takes elements
    // [c*4E, c*4E + 4E) of every row, lane quarter qd = lane / 16 the E of them at
    // c*4E + qd*E. Any split that A and B share gives the same dot products; this one makes
    // every K load instruction read 64 contiguous bytes of each of the 16 rows.
    // Query fragment: lane (column h = lane % 16, quarter qd) holds those elements of
    // q[b, hq0 + h, :]; zero for padded columns h >= G.
    const int col = lane & 15;
    const int qd = lane >> 4;
    u32x4_t qf[NL];
    if (col < G) {
        const char* qrow = p.q + ((int64_t)b * p.Hq + hq0 + col) * D * EB;
#pragma unroll
        for (int c = 0; c < NL; ++c)
            qf[c] = *reinterpret_cast<const u32x4_t*>(qrow + (c * 4 * E + qd * E) * EB);
    } else {
#pragma unroll
        for (int c = 0; c < NL; ++c) qf[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    wave_sync();

    // One stream of 2 * ngroups items: item i < ngroups is K group i, item ngroups + i is
    // V group i. Each item is NL 16-byte loads per lane; a ring of DEPTH items keeps
    // DEPTH * NL * 1 KiB in flight per wave, and V loads are already under way while
    // the softmax statistics of the partition are formed.
    const int64_t head_rows = (int64_t)p.bs;
    const int64_t blk_rows = (int64_t)p.Hkv * head_rows;
    const int bs_mask = p.bs - 1;
    const int lane_k_off = col * ROW + qd * 16;        // K: row `col`, piece `qd` (+64 B per load)
    const int vrow = lane / O;
    const int voct = lane % O;
    const int lane_v_off = vrow * ROW + voct * 16;     // V: row `vrow` (+R per load), slice voct
    const int nitems = 2 * ngroups;

    // Loads are issued unconditionally and in program order (past the end the index is
    // clamped to the last item, a re-read that hits in cache), so the compiler can keep
    // DEPTH - 1 items outstanding while it consumes one.
    auto issue = [&](int item, u32x4_t (&dst)[NL]) {
        item = item < nitems ? item : nitems - 1;
        const bool is_v = item >= ngroups;
        const int tl = (is_v ? item - ngroups : item) << 4;
        const int phys = __builtin_amdgcn_readfirstlane(tbl[tl >> p.bs_shift]);
        const int64_t row0 = (int64_t)phys * blk_rows + g * head_rows + (tl & bs_mask);
        const char* sbase = (is_v ? p.v : p.k) + row0 * ROW;
        const uint32_t voff = is_v ? lane_v_off : lane_k_off;
        const uint32_t vstride = is_v ? R * ROW : 64;
#pragma unroll
        for (int c = 0; c < NL; ++c)
            dst[c] = load16(reinterpret_cast<const u32x4_t*>(sbase + voff + c * vstride));
    };

    u32x4_t ring[DEPTH][NL];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) issue(j, ring[j]);

    float m_run = -INFINITY;
    float l_sum = 0.f;
    float acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;

    for (int i0 = 0; i0 < nitems; i0 += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            const int it = i0 + j;
            if (it < nitems) {
                if (it < ngroups) {
                    // ---- scores of K group `it` on the matrix cores
                    const int tl = it << 4;
                    const f32x4_t sc = qk_tile<BF16, NL>(ring[j], qf);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tl + 4 * qd + i;
                        const float s = (t < ntok) ? sc[i] * p.scale_log2 : -INFINITY;
                        if (col < G) s_lds[t * G + col] = s;
                        m_run = fmaxf(m_run, s);
                    }
                    if (it == ngroups - 1) {
                        // ---- partition statistics: per-head max, p = exp2(s - m), sums
                        m_run = fmaxf(m_run, __shfl_xor(m_run, 16));
                        m_run = fmaxf(m_run, __shfl_xor(m_run, 32));
                        wave_sync();
                        const float m_mine = __shfl(m_run, lane % G);
                        const int nent = ngroups * 16 * G;
                        for (int e = lane; e < nent; e += 64) {
                            const float pe = __builtin_amdgcn_exp2f(s_lds[e] - m_mine);
                            s_lds[e] = pe;
                            l_sum += pe;
                        }
#pragma unroll
                        for (int off = G; off < 64; off <<= 1) l_sum += __shfl_xor(l_sum, off);
                        wave_sync();
                    }
                } else {
                    // ---- o += p * V for V group `it - ngroups` on the vector ALUs
                    const int tl = (it - ngroups) << 4;
                    if (tl + 16 > ntok) {   // last, partly valid group: zero rows past the end
#pragma unroll
                        for (int k = 0; k < NL; ++k)
                            if (tl + vrow + k * R >= ntok) ring[j][k] = u32x4_t{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int k = 0; k < NL; ++k) {
                        float pk[G];
                        load_probs<G>(s_lds + (tl + vrow + k * R) * G, pk);
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const uint32_t u = ring[j][k][w];
                            if constexpr (BF16) {
                                const float x0 = lo_bf16(u), x1 = hi_bf16(u);
#pragma unroll
                                for (int h = 0; h < G; ++h) {
                                    acc[h][2 * w] = fmaf(pk[h], x0, acc[h][2 * w]);
                                    acc[h][2 * w + 1] = fmaf(pk[h], x1, acc[h][2 * w + 1]);
                                }
                            } else {
                                const float x = __uint_as_float(u);
#pragma unroll
                                for (int h = 0; h < G; ++h) acc[h][w] = fmaf(pk[h], x, acc[h][w]);
                            }
                        }
                    }
                }
            }
            issue(it + DEPTH, ring[j]);
        }
    }

    // sum the R row-groups that share a column slice
#pragma unroll
    for (int off = O; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);

    float l_head[G];
#pragma unroll
    for (int h = 0; h < G; ++h) l_head[h] = __shfl(l_sum, h);

    if (nparts_b == 1) {
        if (vrow == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = 1.0f / l_head[h];
                float* dst = p.out + ((int64_t)b * p.Hq + hq0 + h) * D + voct * E;
#pragma unroll
                for (int e = 0; e < E; e += 4)
                    *reinterpret_cast<float4*>(dst + e) =
                        make_float4(acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv,
                                    acc[h][e + 3] * inv);
            }
        }
    } else {
        if (vrow == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float* dst = p.ws_o + (((int64_t)b * p.Hq + hq0 + h) * p.n_parts + part) * D +
                             voct * E;
#pragma unroll
                for (int e = 0; e < E; e += 4)
                    *reinterpret_cast<float4*>(dst + e) =
                        make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
            }
        }
        if (lane < G) {   // lane h holds head h's max (col == h) and sum (h % G == h)
            p.ws_ml[((int64_t)b * p.Hq + hq0 + lane) * p.n_parts + part] = make_float2(m_run, l_sum);
        }
    }
}

// ---------------------------------------------------------------------------------------
// bf16 caches: one pass per partition, K and V of each 16-token group loaded together,
// both contractions on the matrix cores.
//
// QK^T: v_mfma_f32_16x16x32_bf16 with A = the 16 K rows of the group and B = query heads.
// MFMA row m = 4r + i carries token r + 4i (r = lane / 16 of the lane feeding that row
// is not the same r; the permutation only decides which row each lane loads), and the 16
// columns carry the group's 4 heads of a head set, each repeated 4 times. Then lane
// (r = lane / 16, c = lane % 16) receives in register i the score of token r + 4i for head
// c % 4, which is exactly the A operand that v_mfma_f32_4x4x1_16b_f32 (16 blocks of
// 4 x 4 x 1) needs for PV: block lanes 4b..4b+3 (all of row group r) supply
// p[head lane % 4][token r + 4i] and, as B, one element of V row r + 4i, the element a
// coalesced 16-byte load of that row already holds. PV therefore needs no transpose, no
// LDS and no cross-lane exchange; the four row groups' partial sums are added at the end.
//
// Work is done in chunks of kChunk groups (128 tokens): the chunk's kChunk QK^T MFMA
// chains are independent, then one online-softmax update per head (new running maximum,
// accumulators and running sum multiplied by exp2(old max - new max), a factor that is
// exactly 1 when the maximum did not move), then the chunk's PV MFMAs. The loads form one
// stream in consumption order, K of the chunk's groups then V of the same groups, held in
// a ring of DEPTH items of equal size, so DEPTH - 1 items are in flight while one is used.

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int W> struct VecOf;
template <> struct VecOf<16> { typedef u32x4_t type; };
template <> struct VecOf<8> { typedef u32x2_t type; };

// Sum / max over the four 16-lane row groups without LDS traffic: gfx950's permlane swaps
// exchange the odd rows (16 lanes) / the upper half (32 lanes) of one register with the
// even rows / lower half of another. Given two registers holding the same values, they
// then hold the row pairs (0,1),(2,3) crosswise, so one add or max completes a butterfly
// step. Both registers are outputs of the instruction, so it is written as inline
// assembly with two read-write operands (preceded by the wait states a VALU result needs
// before a permlane reads it).
__device__ __forceinline__ void swap_rows16(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float rows_sum(float v) {
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap_rows16(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    uint32_t d = c;
    swap_halves(c, d);
    return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}
__device__ __forceinline__ float rows_max(float v) {
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap_rows16(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    uint32_t d = c;
    swap_halves(c, d);
    return fmaxf(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
// value of lane (lane & ~3) + m of the same quad, via DPP
__device__ __forceinline__ float quad_bcast(float v, int m) {
    const int x = __builtin_bit_cast(int, v);
    int y;
    switch (m) {
        case 0: y = __builtin_amdgcn_mov_dpp(x, 0x00, 0xf, 0xf, false); break;
        case 1: y = __builtin_amdgcn_mov_dpp(x, 0x55, 0xf, 0xf, false); break;
        case 2: y = __builtin_amdgcn_mov_dpp(x, 0xaa, 0xf, 0xf, false); break;
        default: y = __builtin_amdgcn_mov_dpp(x, 0xff, 0xf, 0xf, false); break;
    }
    return __builtin_bit_cast(float, y);
}

template <int D, int G, int DEPTH, int kChunk, bool QLDS>
__global__ __launch_bounds__(64) void decode_bf16_kernel(Params p) {
    constexpr int ROW = D * 2;              // bytes per cached row
    constexpr int NQ = D / 32;              // 16-byte registers per ring item
    constexpr int WV = D / 8;               // bytes of a V row per lane per load (16 or 8)
    constexpr int EV = D / 16;              // bf16 elements per lane per V load
    constexpr int NSET = (G + 3) / 4;       // head sets of 4
    constexpr int G4 = G < 4 ? G : 4;       // distinct heads in a set
    constexpr int ITEMS = 2 * kChunk;       // ring items per chunk: K groups, then V groups
    typedef typename VecOf<WV>::type vload_t;
    static_assert(D == 64 || D == 128, "head size");
    static_assert(kChunk % DEPTH == 0, "the ring depth must divide the chunk");

    const int lane = threadIdx.x;
    int g, b, part;
    work_item(p, g, b, part);
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int hq0 = g * G;
    const int t0 = part * p.part_tokens;
    // The block-table slice of the partition is fetched before the sequence length is
    // known (it does not depend on it): lane i holds entry i, clamped into the row and
    // into the pool, and the loop reads it with v_readlane.
    const int blk0 = t0 >> p.bs_shift;
    int tblv;
    {
        const int32_t* trow = p.tables + (int64_t)b * p.max_blocks;
        int i = blk0 + lane;
        i = i < p.max_blocks ? i : p.max_blocks - 1;
        const int e = trow[i];
        tblv = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
    }
    if (t0 >= L) {
        if (part == 0) {   // empty sequence: a zero row per head
            for (int i = lane; i < G * D; i += 64)
                p.out[((int64_t)b * p.Hq + hq0) * D + i] = 0.f;
        }
        return;
    }
    const int ntok = min(p.part_tokens, L - t0);
    const int ngroups = (ntok + 15) >> 4;
    const int last = ngroups - 1;
    const int nchunks = (ngroups + kChunk - 1) / kChunk;
    const int nparts_b = (L + p.part_tokens - 1) / p.part_tokens;

    const int r = lane >> 4;     // row group
    const int c = lane & 15;     // column
    // query fragments, B operand of QK: column c of set s is head 4s + (c % 4) % G4; held
    // in registers, or (QLDS) parked in LDS and re-read per group to save registers
    u32x4_t qf[QLDS ? 1 : NSET][QLDS ? 1 : NQ];
    __shared__ u32x4_t q_lds[QLDS ? NSET * NQ * 64 : 1];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        const int h = 4 * s + ((c & 3) % G4);
        const char* qrow = p.q + ((int64_t)b * p.Hq + hq0 + h) * ROW;
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + (k * 32 + r * 8) * 2);
            if constexpr (QLDS) q_lds[(s * NQ + k) * 64 + lane] = x;
            else qf[s][k] = x;
        }
    }
    auto qfrag = [&](int s, int k) -> u32x4_t {
        if constexpr (QLDS) return q_lds[(s * NQ + k) * 64 + lane];
        else return qf[s][k];
    };
    if constexpr (QLDS) wave_sync();

    const int64_t tile_bytes = (int64_t)p.bs * ROW;              // one (block, head) tile
    const int64_t blk_bytes = (int64_t)p.Hkv * tile_bytes;       // one physical block
    const char* kbase = p.k + g * tile_bytes;
    const char* vbase = p.v + g * tile_bytes;
    const int bs_mask = p.bs - 1;
    // K: lane feeds MFMA row c, i.e. token (c / 4) + 4 (c % 4) of the group, 16 bytes at
    // 64 k + 16 r; V: row r (+4 per load), bytes c * WV of the row
    const uint32_t koff = (uint32_t)(((c >> 2) + 4 * (c & 3)) * ROW + r * 16);
    const uint32_t voff = (uint32_t)(r * ROW + c * WV);

    struct Item {
        u32x4_t q[NQ];
    };
    // load stream item t of chunk ch (t < kChunk: K of group t, else V of group t - kChunk);
    // groups past the partition are clamped to its last group (a re-read that hits in cache)
    auto issue = [&](int ch, int t, Item& dst) {
        const bool is_v = t >= kChunk;
        int gi = ch * kChunk + (is_v ? t - kChunk : t);
        gi = gi < last ? gi : last;
        const int ph = __builtin_amdgcn_readlane(tblv, (gi << 4) >> p.bs_shift);
        const int64_t off = (int64_t)ph * blk_bytes + (int64_t)((gi << 4) & bs_mask) * ROW;
        if (!is_v) {
            const char* kb = kbase + off;
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                dst.q[k] = *reinterpret_cast<const u32x4_t*>(kb + koff + k * 64);
        } else {
            const char* vb = vbase + off;
            if constexpr (WV == 16) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    dst.q[k] = *reinterpret_cast<const u32x4_t*>(vb + voff + k * 4 * ROW);
            } else {
#pragma unroll
                for (int k = 0; k < 4; k += 2) {
                    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vb + voff + k * 4 * ROW);
                    const u32x2_t e = *reinterpret_cast<const u32x2_t*>(vb + voff + (k + 1) * 4 * ROW);
                    dst.q[k / 2] = __builtin_shufflevector(a, e, 0, 1, 2, 3);
                }
            }
        }
    };
    // dword w of V load k within an item
    auto vword = [&](const Item& it, int k, int w) -> uint32_t {
        if constexpr (WV == 16) return it.q[k][w];
        else return it.q[k >> 1][(k & 1) * 2 + w];
    };

    f32x4_t acc[NSET][EV];
    float m_run[NSET], l_run[NSET];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        m_run[s] = -INFINITY;
        l_run[s] = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[s][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float cl2 = p.scale_log2;

    Item ring[DEPTH];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) issue(0, j, ring[j]);

    // One chunk: consume its 2 * kChunk stream items in order, refilling each ring slot
    // with the item DEPTH positions later. `masked` (the last chunk only) handles tokens
    // past the end of the partition and groups past its last one.
    auto chunk = [&](int ch, bool masked) {
        float y[NSET][kChunk][4];   // scores in log2 units, then probabilities
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            Item& it = ring[t % DEPTH];
            if (t < kChunk) {
                // ---- scores of group t on the matrix cores
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < NQ; ++k)
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, it.q[k]),
                            __builtin_bit_cast(bf16x8_t, qfrag(s, k)), sc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[s][t][i] = sc[i] * cl2;
                }
                if (t == kChunk - 1) {
                    // ---- one online-softmax update for the chunk's 128 tokens
                    const int tc = ch * kChunk * 16;   // first token of the chunk
#pragma unroll
                    for (int s = 0; s < NSET; ++s) {
                        if (masked) {
#pragma unroll
                            for (int u = 0; u < kChunk; ++u)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    y[s][u][i] = (tc + u * 16 + r + 4 * i < ntok) ? y[s][u][i] : -INFINITY;
                        }
                        float mx = y[s][0][0];
#pragma unroll
                        for (int u = 0; u < kChunk; ++u)
#pragma unroll
                            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, y[s][u][i]);
                        const float m_new = fmaxf(m_run[s], rows_max(mx));
                        const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
                        m_run[s] = m_new;
                        float am[4];
#pragma unroll
                        for (int m = 0; m < 4; ++m) am[m] = quad_bcast(alpha, m);
#pragma unroll
                        for (int e = 0; e < EV; ++e)
#pragma unroll
                            for (int m = 0; m < 4; ++m) acc[s][e][m] *= am[m];
                        float ls = 0.f;
#pragma unroll
                        for (int u = 0; u < kChunk; ++u) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float e2 = __builtin_amdgcn_exp2f(y[s][u][i] - m_new);
                                y[s][u][i] = masked ? ((y[s][u][i] == -INFINITY) ? 0.f : e2) : e2;
                            }
                            ls += (y[s][u][0] + y[s][u][1]) + (y[s][u][2] + y[s][u][3]);
                        }
                        l_run[s] = l_run[s] * alpha + ls;
                    }
                }
            } else {
                // ---- o += p * V for group u on the matrix cores
                const int u = t - kChunk;
                const int gi = ch * kChunk + u;
                bool skip = false;
                if (masked) {
                    skip = gi > last;
                    if (!skip && gi == last) {   // rows past the end may hold anything
                        const int tl = gi * 16;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            if (tl + r + 4 * k >= ntok) {
                                if constexpr (WV == 16) {
                                    it.q[k] = u32x4_t{0u, 0u, 0u, 0u};
                                } else {
                                    it.q[k >> 1][(k & 1) * 2] = 0u;
                                    it.q[k >> 1][(k & 1) * 2 + 1] = 0u;
                                }
                            }
                        }
                    }
                }
                if (!skip) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
#pragma unroll
                        for (int w = 0; w < WV / 4; ++w) {
                            const uint32_t uw = vword(it, k, w);
                            const float v0 = lo_bf16(uw), v1 = hi_bf16(uw);
#pragma unroll
                            for (int s = 0; s < NSET; ++s) {
                                acc[s][2 * w] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[s][u][k], v0, acc[s][2 * w], 0, 0, 0);
                                acc[s][2 * w + 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[s][u][k], v1, acc[s][2 * w + 1], 0, 0, 0);
                            }
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue(ch + (t + DEPTH) / ITEMS, (t + DEPTH) % ITEMS, it);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int ch = 0; ch < nchunks - 1; ++ch) chunk(ch, false);
    chunk(nchunks - 1, true);

    // add the four row groups' partial sums (lanes c, c + 16, c + 32, c + 48)
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        l_run[s] = rows_sum(l_run[s]);
#pragma unroll
        for (int e = 0; e < EV; ++e)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[s][e][m] = rows_sum(acc[s][e][m]);
    }
    // lane c (row group 0) now holds, for head m of each set, output columns
    // c*EV .. c*EV+EV-1; head m's sum and running maximum sit in quad lane m
    float lh[NSET][4], mh[NSET][4];
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            lh[s][m] = quad_bcast(l_run[s], m);
            mh[s][m] = quad_bcast(m_run[s], m);
        }
    if (r == 0) {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
#pragma unroll
            for (int m = 0; m < G4; ++m) {
                const int h = 4 * s + m;
                float o[EV];
#pragma unroll
                for (int e = 0; e < EV; ++e) o[e] = acc[s][e][m];
                if (nparts_b == 1) {
                    const float inv = 1.0f / lh[s][m];
                    float* dst = p.out + ((int64_t)b * p.Hq + hq0 + h) * D + c * EV;
#pragma unroll
                    for (int e = 0; e < EV; e += 4)
                        *reinterpret_cast<float4*>(dst + e) =
                            make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
                } else {
                    float* dst = p.ws_o + (((int64_t)b * p.Hq + hq0 + h) * p.n_parts + part) * D + c * EV;
#pragma unroll
                    for (int e = 0; e < EV; e += 4)
                        *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                    if (c == 0)
                        p.ws_ml[((int64_t)b * p.Hq + hq0 + h) * p.n_parts + part] =
                            make_float2(mh[s][m], lh[s][m]);
                }
            }
        }
    }
}

// Combine the partitions of one (sequence, query head):
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, with M = max_i m_i.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(Params p) {
    constexpr int C4 = D / 4;          // float4 columns
    constexpr int NPG = 256 / C4;      // partition groups per block
    __shared__ float red_m[4];
    __shared__ float4 red_o[NPG][C4];
    __shared__ float red_l[NPG];

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int np = (L + p.part_tokens - 1) / p.part_tokens;
    if (np <= 1) return;
    const int64_t row = (int64_t)b * p.Hq + h;
    const float2* ml = p.ws_ml + row * p.n_parts;
    const float* wo = p.ws_o + row * p.n_parts * D;

    float mx = -INFINITY;
    for (int i = tid; i < np; i += 256) mx = fmaxf(mx, ml[i].x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) red_m[tid >> 6] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

    const int c4 = tid % C4;
    const int pg = tid / C4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int i = pg; i < np; i += NPG) {
        const float2 mli = ml[i];
        const float w = __builtin_amdgcn_exp2f(mli.x - M);
        const float4 o = reinterpret_cast<const float4*>(wo + (int64_t)i * D)[c4];
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
        den = fmaf(w, mli.y, den);
    }
    red_o[pg][c4] = acc;
    if (c4 == 0) red_l[pg] = den;
    __syncthreads();
    if (pg == 0) {
        float4 s = red_o[0][c4];
        float dsum = red_l[0];
        for (int j = 1; j < NPG; ++j) {
            const float4 x = red_o[j][c4];
            s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
            dsum += red_l[j];
        }
        const float inv = 1.0f / dsum;
        reinterpret_cast<float4*>(p.out + row * D)[c4] =
            make_float4(s.x * inv, s.y * inv, s.z * inv, s.w * inv);
    }
}



template <bool BF16, int D, int G>
hipError_t launch_one(const Params& prm, int B, int Hkv, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if constexpr (BF16) {
        hipLaunchKernelGGL((decode_bf16_kernel<D, G, PA_BF16_DEPTH, PA_BF16_CHUNK, (PA_BF16_QLDS != 0)>), dim3(prm.n_parts * Hkv * B),
                           dim3(64), 0, s, prm);
    } else {
        const size_t lds = (size_t)prm.part_tokens * G * sizeof(float) +
                           (size_t)(prm.part_tokens / 16) * sizeof(int);
        hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G, PA_DECODE_DEPTH>),
                           dim3(prm.n_parts * Hkv * B), dim3(64), lds, s, prm);
    }
    if (prm.n_parts > 1)
        hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(prm.Hq, B), dim3(256), 0, s, prm);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t dispatch_g(const Params& prm, int B, int Hkv, int G, void* stream) {
    switch (G) {
        case 1: return launch_one<BF16, D, 1>(prm, B, Hkv, stream);
        case 2: return launch_one<BF16, D, 2>(prm, B, Hkv, stream);
        case 4: return launch_one<BF16, D, 4>(prm, B, Hkv, stream);
        case 8: return launch_one<BF16, D, 8>(prm, B, Hkv, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t dispatch_d(const Params& prm, int B, int Hkv, int D, int G, void* stream) {
    if (D == 64) return dispatch_g<BF16, 64>(prm, B, Hkv, G, stream);
    if (D == 128) return dispatch_g<BF16, 128>(prm, B, Hkv, G, stream);
    return hipErrorInvalidValue;
}

}  // namespace

namespace pa_internal {

int launch_decode(const DecodeLaunch& a, const char** err) {
    Params prm;
    prm.out = a.out;
    prm.ws_o = a.ws_o;
    prm.ws_ml = reinterpret_cast<float2*>(a.ws_ml);
    prm.q = static_cast<const char*>(a.q);
    prm.k = static_cast<const char*>(a.k);
    prm.v = static_cast<const char*>(a.v);
    prm.tables = a.tables;
    prm.lens = a.lens;
    prm.B = a.B;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.bs = a.bs;
    int shift = 0;
    while ((1 << shift) < a.bs) ++shift;
    prm.bs_shift = shift;
    prm.num_blocks = a.num_blocks;
    prm.max_blocks = a.max_blocks;
    prm.part_tokens = a.part_tokens;
    prm.n_parts = a.n_parts;
    prm.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    (void)kLog2e;
    if (a.B == 0) return 0;
    const int G = a.Hq / a.Hkv;
    hipError_t e = a.kv_dtype == 1 ? dispatch_d<true>(prm, a.B, a.Hkv, a.D, G, a.stream)
                                   : dispatch_d<false>(prm, a.B, a.Hkv, a.D, G, a.stream);
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

}  // namespace pa_internal
