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
    int Hq, Hkv, bs, bs_shift, num_blocks, max_blocks, part_tokens, n_parts;
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

template <bool BF16, int D, int G>
__global__ __launch_bounds__(64) void decode_partition_kernel(Params p) {
    constexpr int EB = BF16 ? 2 : 4;   // bytes per element
    constexpr int E = 16 / EB;         // elements per 16-byte load
    constexpr int KQ = D / 4;          // elements of a K row fed by one lane (quarter row)
    constexpr int KL = KQ / E;         // 16-byte loads per lane per 16-token K group
    constexpr int O = D / E;           // lanes covering one V row
    constexpr int R = 64 / O;          // V rows per wave-wide load
    constexpr int VL = 16 / R;         // wave-wide V loads per 16-token group
    constexpr int ROW = D * EB;        // bytes per cached row
    static_assert(KL >= 1 && R >= 1 && VL >= 1, "unsupported head size");

    extern __shared__ float smem[];
    float* s_lds = smem;                                  // [part_tokens][G]
    int* tbl = reinterpret_cast<int*>(smem + p.part_tokens * G);   // [part_tokens / 16]

    const int lane = threadIdx.x;
    const int part = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
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

    // query fragment: lane (column h = lane % 16, quarter qd = lane / 16) holds
    // q[b, hq0 + h, qd*KQ .. qd*KQ + KQ); zero for padded columns h >= G
    const int col = lane & 15;
    const int qd = lane >> 4;
    u32x4_t qf[KL];
    if (col < G) {
        const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(
            p.q + (((int64_t)b * p.Hq + hq0 + col) * D + qd * KQ) * EB);
#pragma unroll
        for (int c = 0; c < KL; ++c) qf[c] = qsrc[c];
    } else {
#pragma unroll
        for (int c = 0; c < KL; ++c) qf[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    const int64_t head_rows = (int64_t)p.bs;              // rows per (block, head) tile
    const int64_t blk_rows = (int64_t)p.Hkv * head_rows;  // rows per physical block
    const int bs_mask = p.bs - 1;

    // ---- pass 1: scores
    float m_run = -INFINITY;
    const int lane_k_off = col * ROW + qd * KQ * EB;   // this lane's K row quarter
#pragma unroll 2
    for (int gi = 0; gi < ngroups; ++gi) {
        const int tl = gi << 4;
        const int phys = __builtin_amdgcn_readfirstlane(tbl[tl >> p.bs_shift]);
        const int64_t row0 = (int64_t)phys * blk_rows + g * head_rows + (tl & bs_mask);
        const u32x4_t* ksrc = reinterpret_cast<const u32x4_t*>(p.k + row0 * ROW + lane_k_off);
        u32x4_t kf[KL];
#pragma unroll
        for (int c = 0; c < KL; ++c) kf[c] = __builtin_nontemporal_load(ksrc + c);
        const f32x4_t sc = qk_tile<BF16, KL>(kf, qf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tl + 4 * qd + i;
            const float s = (t < ntok) ? sc[i] * p.scale_log2 : -INFINITY;
            if (col < G) s_lds[t * G + col] = s;
            m_run = fmaxf(m_run, s);
        }
    }
    // lanes col, col+16, col+32, col+48 hold the same head
    m_run = fmaxf(m_run, __shfl_xor(m_run, 16));
    m_run = fmaxf(m_run, __shfl_xor(m_run, 32));
    __syncthreads();

    // ---- pass 2: probabilities in place, per-head sums (lane handles head lane % G)
    const float m_mine = __shfl(m_run, lane % G);
    float l_sum = 0.f;
    const int nent = ngroups * 16 * G;
    for (int e = lane; e < nent; e += 64) {
        const float pe = __builtin_amdgcn_exp2f(s_lds[e] - m_mine);
        s_lds[e] = pe;
        l_sum += pe;
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) l_sum += __shfl_xor(l_sum, off);
    __syncthreads();

    // ---- pass 3: o = sum_t p_t v_t
    const int vrow = lane / O;
    const int voct = lane % O;
    float acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    const int lane_v_off = vrow * ROW + voct * 16;
#pragma unroll 2
    for (int gi = 0; gi < ngroups; ++gi) {
        const int tl = gi << 4;
        const int phys = __builtin_amdgcn_readfirstlane(tbl[tl >> p.bs_shift]);
        const int64_t row0 = (int64_t)phys * blk_rows + g * head_rows + (tl & bs_mask);
        const char* vsrc = p.v + row0 * ROW + lane_v_off;
        u32x4_t vf[VL];
#pragma unroll
        for (int k = 0; k < VL; ++k)
            vf[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vsrc + k * R * ROW));
        if (tl + 16 > ntok) {   // last, partly valid group: zero rows past the end
#pragma unroll
            for (int k = 0; k < VL; ++k)
                if (tl + vrow + k * R >= ntok) vf[k] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < VL; ++k) {
            float pk[G];
            load_probs<G>(s_lds + (tl + vrow + k * R) * G, pk);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t u = vf[k][w];
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
    const size_t lds = (size_t)prm.part_tokens * G * sizeof(float) +
                       (size_t)(prm.part_tokens / 16) * sizeof(int);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G>), dim3(prm.n_parts, Hkv, B), dim3(64),
                       lds, s, prm);
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
