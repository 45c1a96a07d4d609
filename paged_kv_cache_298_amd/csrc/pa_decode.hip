// pa_decode.hip -- paged decode attention for gfx950 (MI355X).
//
// Sources: [P1] "PagedAttention" (inferensys.com glossary): the kernel reads the block
// table, gathers K/V from scattered physical blocks, handles a partly filled last block
// and fuses the gather into the attention; [P2] "Paged Attention" tutorial
// (infra.pidoku.co.in), section 5 "The kernel side": a loop over a sequence's blocks,
// phys = table[blk], q.k and an online softmax accumulated per block. That page's sketch
// and its cache layouts were written for NVIDIA warps; this file keeps what it computes
// and lays the work out for 64-lane CDNA4 wavefronts.
//
// Cache layout [num_blocks, Hkv, block_size, D]: a 16-token group of one KV head is one
// contiguous 16 x D tile of K and one of V. Every wavefront serves all G = Hq / Hkv query
// heads of its KV head, so each K/V byte is read from HBM once.
//
// Kernels:
//   decode_stream_kernel + stream_reduce_kernel (bf16 caches, the default): the batch's
//     (sequence, KV head) rows, cut into 16-token groups, are laid end to end and each
//     resident wavefront takes an equal contiguous slice; one load ring runs across row
//     boundaries; rows that cross slices leave partial states merged by the second kernel.
//   decode_bf16_kernel (bf16 fallback) and decode_partition_kernel (fp32): one workgroup
//     per (KV head, sequence, partition of P tokens); decode_reduce_kernel merges the
//     partitions.
// Scores: v_mfma_f32_16x16x32_bf16 (fp32: 16x16x4_f32) with the K tile as the A operand,
// each lane feeding token (c / 4) + 4 (c % 4) of its row group straight from one 16-byte
// load, and the G query rows (replicated to 16 columns) as B; lane (r, c) then holds
// tokens r + 4i of head column c. Softmax: online, in log2 units, masks by select (NaN in
// unused slots never leaks). PV: the stream kernel feeds those same registers (rounded to
// bf16) as the A operand of v_mfma_f32_16x16x16_bf16 against V rows gathered with byte
// permutes; the bf16 partition kernel uses v_mfma_f32_4x4x1_f32, the fp32 one the VALU.
#include <mutex>

#include "pa_device.h"

namespace {

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
    work_item(p, blockIdx.x, g, b, part);
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

template <int D, int G, int DEPTH, int kChunk, bool QLDS, int W>
__global__ __launch_bounds__(64 * W) void decode_bf16_kernel(Params p) {
    bf16_item<D, G, DEPTH, kChunk, QLDS, W>(p, blockIdx.x);
}

// ---------------------------------------------------------------------------------------
// Stream decomposition (bf16 KV). The rows (sequence b, KV head g), each cut into
// ceil(L_b / 16) groups of 16 tokens, are laid end to end into one stream of T groups,
// and each of nw resident waves takes an equal contiguous slice of it. A wave walks its
// slice with one load ring that never drains between rows: it finishes rows it covers
// whole by writing the output directly, and leaves a partial state (max, sum, unscaled
// output) for the at most two rows it covers only in part; stream_reduce_kernel merges
// those. Each group's K tile and V tile are 4 KiB items of the ring; the online softmax
// is updated once per group. Block-table lookups for 64 groups at a time ("window") are
// resolved lane-parallel: lane i finds the row of group sw + i by a binary search over
// the per-sequence prefix of group counts kept in LDS, then gathers its table entry.
// SPLIT: blocks of 8 tokens, so a 16-token group spans two physical blocks; each group
// then has two tile offsets (tokens 0-7 and 8-15) and K lanes / V loads pick theirs.
// FUSED (pa_decode_append): the batch's newest tokens are also written to their slots by
// this launch (the reshape_and_cache step); the lanes that would read position L - 1 of a
// sequence with a new token read it from the input rows instead, so no wave reads a slot
// written in the same launch and the result is that of the write followed by the decode.
template <int D, int G, int DEPTH, bool SPLIT, bool MULTI, bool DIST, bool FUSED = false>
__global__ __launch_bounds__(256) void decode_stream_kernel(Params p) {
    constexpr int ROW = D * 2;              // bytes per cached row
    constexpr int NQ = D / 32;              // 16-byte registers per ring item
    constexpr int WV = D / 8;               // bytes of a V row per lane per load (16 or 8)
    constexpr int EV = D / 16;              // bf16 elements per lane per V load
    // head sets of 4, each head repeated over the 16 columns; COLS (MULTI, or DIST for a
    // decode with G = 8): one set whose 16 columns hold the G (4, 8 or 16) query columns,
    // repeated 16 / G times, so that output row 4r + i of the PV tile is column 4r + i
    constexpr bool COLS = MULTI || DIST;
    static_assert(!COLS || G == 4 || G == 8 || G == 16, "columns of one tile");
    constexpr int NSET = COLS ? 1 : (G + 3) / 4;
    constexpr int G4 = G < 4 ? G : 4;       // distinct heads in a set
    constexpr int U = DEPTH / 2;            // groups in flight ahead of the consumer
    static_assert(D == 64 || D == 128, "head size");
    static_assert(DEPTH >= 2 && DEPTH % 2 == 0, "ring holds whole groups (K and V)");
    // MULTI: G counts query columns, token j of the sequence's last n (its queries) times
    // the GK heads of the KV head (column h = j GK + head); a row with no queries is empty
    const int GK = MULTI ? p.Hq / p.Hkv : G;

    extern __shared__ int lds_prefix[];
    int* Cs = lds_prefix;           // [B + 1] exclusive prefix of groups per sequence
    int* Ls = lds_prefix + p.B + 1; // [B] lengths clamped into the table's capacity
    int* Ns = Ls + p.B;             // FUSED: [B] 1 when the sequence's newest token is given
    __shared__ int wsum[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cap = p.max_blocks * p.bs;

    // FUSED: the cache write. (sequence, KV head) row r of the new tokens goes to its slot,
    // rows gw, gw + nw, ... per wave (lanes 0 .. ROW/16-1 move K, the next ROW/16 lanes V).
    // The first row's load is issued here, beside the lengths' loads, and stored once they
    // are in, so the write adds no round trip ahead of the first K/V tile.
    constexpr int UR = ROW / 16;
    const int gw0 = blockIdx.x * 4 + wid;
    const bool cw_lane = lane < 2 * UR;
    const bool cw_v = lane >= UR;
    const int cw_u = cw_v ? lane - UR : lane;
    // the destination of row r, whose sequence's slot is sl (-1: no write)
    auto cw_dst = [&](int r, int sl) -> int64_t {
        const int g = r - (r / p.Hkv) * p.Hkv;
        if (sl < 0 || (int64_t)sl >= (int64_t)p.num_blocks * p.bs) return -1;
        return (((int64_t)(sl >> p.bs_shift) * p.Hkv + g) * p.bs + (sl & (p.bs - 1))) * ROW + cw_u * 16;
    };
    auto cw_src = [&](int r) -> const u32x4_t* {
        return reinterpret_cast<const u32x4_t*>((cw_v ? p.nval : p.nkey) + (int64_t)r * ROW + cw_u * 16);
    };
    u32x4_t cw_x = {0u, 0u, 0u, 0u};
    int cw_sl = -1;
    if constexpr (FUSED) {
        if (gw0 < p.B * p.Hkv && cw_lane) {   // loads only: their values are used after the prefix
            cw_sl = p.nslots[gw0 / p.Hkv];
            cw_x = *cw_src(gw0);
        }
    }

    // ---- groups per sequence and their exclusive prefix over the batch (whole block)
    const int per = (p.B + 255) >> 8;
    int loc = 0;
    for (int i = 0; i < per; ++i) {
        const int bb = tid * per + i;
        if (bb < p.B) {
            int L = p.lens[bb];
            const int nsl = FUSED ? p.nslots[bb] : -1;   // loaded beside the length
            L = L < 0 ? 0 : (L > cap ? cap : L);
            if constexpr (MULTI) {
                int qs_, n_;
                multi_rows(p, bb, L, &qs_, &n_);
                L = n_ > 0 ? L : 0;
            }
            Ls[bb] = L;
            if constexpr (FUSED) Ns[bb] = (L > 0 && nsl >= 0) ? 1 : 0;
            loc += (L + 15) >> 4;
        }
    }
    int inc = loc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d);
        if (lane >= d) inc += y;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int run = inc - loc;
    for (int v = 0; v < wid; ++v) run += wsum[v];
    for (int i = 0; i < per; ++i) {
        const int bb = tid * per + i;
        if (bb < p.B) {
            Cs[bb] = run;
            run += (Ls[bb] + 15) >> 4;
        }
    }
    if (tid == 255) Cs[p.B] = run;
    __syncthreads();
    if constexpr (FUSED) {
        char* cw_cache = const_cast<char*>(cw_v ? p.v : p.k);
        if (gw0 < p.B * p.Hkv && cw_lane) {
            const int64_t d = cw_dst(gw0, cw_sl);
            if (d >= 0) *reinterpret_cast<u32x4_t*>(cw_cache + d) = cw_x;
        }
        for (int r = gw0 + p.nw; r < p.B * p.Hkv; r += p.nw) {   // more rows than waves
            if (cw_lane) {
                const int64_t d = cw_dst(r, p.nslots[r / p.Hkv]);
                if (d >= 0) *reinterpret_cast<u32x4_t*>(cw_cache + d) = *cw_src(r);
            }
        }
    }

    const int T = __builtin_amdgcn_readfirstlane(Cs[p.B]) * p.Hkv;
    const int gw = blockIdx.x * 4 + wid;
    int nwe = T / p.min_slice;
    nwe = nwe < 1 ? 1 : (nwe > p.nw ? p.nw : nwe);
    if (T == 0) nwe = 0;
    if (gw == 0 && lane == 0) {
        p.meta[0] = T;
        p.meta[1] = nwe;
    }
    // empty sequences: a zero row per query head (MULTI: an empty row has no queries)
    for (int bb = gw; bb < (MULTI ? 0 : p.B); bb += p.nw) {
        if (__builtin_amdgcn_readfirstlane(Ls[bb]) == 0) {
            float* o = p.out + (int64_t)bb * p.Hq * D;
            for (int i = lane; i < p.Hq * D; i += 64) o[i] = 0.f;
        }
    }
    if (gw >= nwe) return;
    const int s0 = (int)((int64_t)gw * T / nwe);
    const int s1 = (int)((int64_t)(gw + 1) * T / nwe);
    const int ns = s1 - s0;

    const int64_t tile_bytes = (int64_t)p.bs * ROW;              // one (block, head) tile
    const int64_t blk_bytes = (int64_t)p.Hkv * tile_bytes;       // one physical block
    const int bs_mask = p.bs - 1;

    // ---- window: lane i describes group sw + i of the slice (clamped into it)
    uint32_t w_lo = 0, w_hi = 0;   // byte offset of the group's tile in either cache
    uint32_t w_lo1 = 0, w_hi1 = 0; // SPLIT: offset of the tile holding tokens 8-15
    int w_row = 0, w_j = 0;        // its row (b * Hkv + g) and group within the row
    int w_new = 0;                 // FUSED: 16 + (L - 1) % 16 when the group holds a given
                                   // newest token at position L - 1, else 0
    int sw = s0;
    auto window = [&](int base) {
        int s = base + lane;
        s = s < s1 ? s : s1 - 1;
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {           // first sequence whose groups end past s
            const int mid = (lo + hi) >> 1;
            if (Cs[mid + 1] * p.Hkv > s) hi = mid;
            else lo = mid + 1;
        }
        const int n = Cs[lo + 1] - Cs[lo];
        const int off = s - Cs[lo] * p.Hkv;
        const int g = off / n;
        const int j = off - g * n;
        const int32_t* trow = p.tables + (int64_t)lo * p.max_blocks;
        int e = trow[(j << 4) >> p.bs_shift];
        e = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
        const int64_t o = (int64_t)e * blk_bytes + (int64_t)g * tile_bytes +
                          (int64_t)((j << 4) & bs_mask) * ROW;
        w_lo = (uint32_t)o;
        w_hi = (uint32_t)((uint64_t)o >> 32);
        if constexpr (SPLIT) {     // the second block of the group (clamped into the row)
            int i1 = 2 * j + 1;
            i1 = i1 < p.max_blocks ? i1 : p.max_blocks - 1;
            int e1 = trow[i1];
            e1 = e1 < 0 ? 0 : (e1 >= p.num_blocks ? p.num_blocks - 1 : e1);
            const int64_t o1 = (int64_t)e1 * blk_bytes + (int64_t)g * tile_bytes;
            w_lo1 = (uint32_t)o1;
            w_hi1 = (uint32_t)((uint64_t)o1 >> 32);
        }
        w_row = lo * p.Hkv + g;
        w_j = j;
        if constexpr (FUSED) w_new = (Ns[lo] != 0 && j == n - 1) ? 16 + ((Ls[lo] - 1) & 15) : 0;
    };
    window(sw);

    // ---- consumer cursor (wave-uniform, kept in scalar registers): sequence, KV head,
    // group in row, groups in row, tokens in row. Lengths are re-read through the scalar
    // cache so that no vector register enters the cursor's updates.
    typedef __attribute__((address_space(4))) const int32_t* const_i32p;
    const const_i32p slens = (const_i32p)(p.lens);
    const const_i32p sqs = (const_i32p)(p.q_starts);
    // MULTI: first query row and query count of sequence bb, clamped as multi_rows does
    auto seq_queries = [&](int bb, int L, int* qs, int* n) {
        int a = sqs[bb];
        a = a < 0 ? 0 : (a > p.total_q ? p.total_q : a);
        int m = sqs[bb + 1] - a;
        m = m < 0 ? 0 : m;
        m = min(m, min(L, p.max_q));
        *qs = a;
        *n = min(m, p.total_q - a);
    };
    auto seq_len = [&](int bb) -> int {
        int L = slens[bb];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        if constexpr (MULTI) {
            int qs_, n_;
            seq_queries(bb, L, &qs_, &n_);
            L = n_ > 0 ? L : 0;
        }
        return L;
    };
    const int row0 = __builtin_amdgcn_readlane(w_row, 0);
    int cb = row0 / p.Hkv;
    int cg = row0 - cb * p.Hkv;
    int cj = __builtin_amdgcn_readlane(w_j, 0);
    int cL = seq_len(cb);
    int cn = (cL + 15) >> 4;
    int cqs = 0, cnq = 0;            // MULTI: the current row's first query and query count
    if constexpr (MULTI) seq_queries(cb, cL, &cqs, &cnq);
    if (lane == 0) p.desc[gw] = make_int4(cb, cg, s0 - cj, cn);

    const int r = lane >> 4;     // row group
    const int c = lane & 15;     // column
    // query fragments of the current row and of the next row the loads reach
    u32x4_t qf[NSET][NQ], qn[NSET][NQ];
    auto load_q = [&](int row, u32x4_t (&dst)[NSET][NQ]) {
        const int bq = row / p.Hkv;
        const int gq = row - bq * p.Hkv;
        int qs = 0, nq = 0;
        if constexpr (MULTI) seq_queries(bq, seq_len(bq), &qs, &nq);
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            const int h = COLS ? c % G : 4 * s + ((c & 3) % G4);
            const char* qrow;
            if constexpr (MULTI) {
                // column h = j GK + head; columns past the row's queries repeat its last
                int j = h / GK;
                j = j < nq ? j : nq - 1;
                j = j < 0 ? 0 : j;
                if (nq == 0) qs = 0;        // not reached for a row in the stream
                qrow = p.q + ((int64_t)(qs + j) * p.Hq + gq * GK + (h - (h / GK) * GK)) * ROW;
            } else {
                qrow = p.q + ((int64_t)bq * p.Hq + gq * G + h) * ROW;
            }
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                dst[s][k] = *reinterpret_cast<const u32x4_t*>(qrow + (k * 32 + r * 8) * 2);
        }
    };
    load_q(row0, qf);
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int k = 0; k < NQ; ++k) qn[s][k] = qf[s][k];
    int qn_row = -1;       // row whose fragments sit in qn
    int iss_row = row0;    // row of the last K tile issued

    // K: lane c of a row group feeds token (c / 4) + 4 (c % 4) of the group; with SPLIT,
    // tokens 8-15 (c % 4 >= 2) come from the second block, at row token - 8
    const int ktok = (c >> 2) + 4 * (c & 3);
    const bool khi = SPLIT && ktok >= 8;
    const uint32_t koff = (uint32_t)((SPLIT ? (ktok & 7) : ktok) * ROW + r * 16);
    const uint32_t voff = (uint32_t)(r * ROW + c * WV);
    struct Item {
        u32x4_t q[NQ];
    };
    // Groups past the slice (the ring runs DEPTH / 2 groups ahead of the consumer) are
    // parked on the first tile of the caches: the data are never used, and one small tile
    // that every wave reads stays in cache, where a re-read of the slice's last group would
    // fetch it from HBM again (the loads are non-temporal).
    auto tile_off = [&](int gq) -> uint64_t {
        int s = s0 + gq;
        if (s >= s1) return 0;
        if (s - sw >= 64) {
            sw += 64;
            window(sw);
        }
        const int idx = s - sw;
        // readlane returns int: through uint32_t, so that a low word with bit 31 set is not
        // sign-extended into the high word (tiles past 2 GiB of a cache)
        return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(w_hi, idx) << 32) |
               (uint64_t)(uint32_t)__builtin_amdgcn_readlane(w_lo, idx);
    };
    // SPLIT: the second block's tile of the same group (the window is already in place)
    auto tile_off1 = [&](int gq) -> uint64_t {
        int s = s0 + gq;
        if (s >= s1) return 0;
        const int idx = s - sw;
        return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(w_hi1, idx) << 32) |
               (uint64_t)(uint32_t)__builtin_amdgcn_readlane(w_lo1, idx);
    };
    auto issue_k = [&](int gq, Item& dst) {
        const uint64_t off = tile_off(gq);
        int s = s0 + gq;
        s = s < s1 ? s : s1 - 1;
        const int row = __builtin_amdgcn_readlane(w_row, s - sw);
        if (row != iss_row) {       // the loads enter a new row: fetch its query early
            iss_row = row;
            qn_row = row;
            load_q(row, qn);
        }
        const char* kb = p.k + off;
        if constexpr (SPLIT) {
            const char* kb1 = p.k + tile_off1(gq);
            kb = khi ? kb1 : kb;
        }
        kb += koff;
        if constexpr (FUSED) {   // the lanes of a given newest token read the input row
            const int nw_info = __builtin_amdgcn_readlane(w_new, s - sw);
            if (nw_info != 0) {   // wave-uniform, a row's last group only; no load inside
                const char* in = p.nkey + (int64_t)row * ROW + r * 16;
                kb = ktok == nw_info - 16 ? in : kb;
            }
        }
#pragma unroll
        for (int k = 0; k < NQ; ++k)
            dst.q[k] = kv_load16(reinterpret_cast<const u32x4_t*>(kb + k * 64));
    };
    // V load k holds rows r + 4k; with SPLIT, loads 2 and 3 (rows 8-15) read the second
    // block at rows r + 4 (k - 2)
    auto issue_v = [&](int gq, Item& dst) {
        const char* vb = p.v + tile_off(gq);
        const char* vb1 = vb + 2 * 4 * ROW;
        if constexpr (SPLIT) vb1 = p.v + tile_off1(gq);
        // address of V load k (rows r + 4k of the group)
        const char* va[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) va[k] = k < 2 ? vb + voff + k * 4 * ROW : vb1 + voff + (k - 2) * 4 * ROW;
        if constexpr (FUSED) {   // the lanes of a given newest token read the input row
            int sv = s0 + gq;
            sv = sv < s1 ? sv : s1 - 1;
            const int nw_info = __builtin_amdgcn_readlane(w_new, sv - sw);
            if (nw_info != 0) {   // wave-uniform, a row's last group only; no load inside
                const char* vin = p.nval + (int64_t)__builtin_amdgcn_readlane(w_row, sv - sw) * ROW + c * WV;
#pragma unroll
                for (int k = 0; k < 4; ++k) va[k] = r + 4 * k == nw_info - 16 ? vin : va[k];
            }
        }
        auto vaddr = [&](int k) -> const char* { return va[k]; };
        if constexpr (WV == 16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst.q[k] = kv_load16(reinterpret_cast<const u32x4_t*>(vaddr(k)));
        } else {
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vaddr(k));
                const u32x2_t e = *reinterpret_cast<const u32x2_t*>(vaddr(k + 1));
                dst.q[k / 2] = __builtin_shufflevector(a, e, 0, 1, 2, 3);
            }
        }
    };
    auto vword = [&](const Item& it, int k, int w) -> uint32_t {
        if constexpr (WV == 16) return it.q[k][w];
        else return it.q[k >> 1][(k & 1) * 2 + w];
    };

    f32x4_t acc[NSET][EV];
    float m_run[NSET], l_run[NSET];
    auto reset = [&]() {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            m_run[s] = -INFINITY;
            l_run[s] = 0.f;
#pragma unroll
            for (int e = 0; e < EV; ++e) acc[s][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    reset();
    bool first_seg = true;   // the slice's first row segment
    int seg_j0 = cj;         // first group of the current row segment
    const float cl2 = p.scale_log2;

    // write the state of the current row segment: the output if the segment is the whole
    // row, else a partial record (slot 0: the slice's first segment, slot 1: its last)
    auto flush = [&]() {
        const bool whole = seg_j0 == 0 && cj == cn - 1;
        float lh[NSET][4], mh[NSET][4];
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            l_run[s] = rows_sum(l_run[s]);   // the output tile needs no sum: rows repeat
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // output row 4r + m holds column 4r + m (COLS), else head m
                lh[s][m] = COLS ? __shfl(l_run[s], 4 * r + m) : quad_bcast(l_run[s], m);
                mh[s][m] = COLS ? __shfl(m_run[s], 4 * r + m) : quad_bcast(m_run[s], m);
            }
        }
        // the row groups holding distinct outputs: one (rows repeat the heads), COLS G / 4
        if (COLS ? 4 * r < G : r == 0) {
            const int rec = 2 * gw + (first_seg ? 0 : 1);
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
#pragma unroll
                for (int m = 0; m < G4; ++m) {
                    const int h = COLS ? 4 * r + m : 4 * s + m;
                    if (whole) {
                        const float inv = 1.0f / lh[s][m];
                        int64_t orow = (int64_t)cb * p.Hq + cg * G + h;
                        if constexpr (MULTI) {
                            const int j = h / GK;
                            if (j >= cnq) continue;          // no such query in this row
                            orow = (int64_t)(cqs + j) * p.Hq + cg * GK + (h - j * GK);
                        }
                        float* dst = p.out + orow * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(acc[s][e][m] * inv, acc[s][e + 1][m] * inv,
                                            acc[s][e + 2][m] * inv, acc[s][e + 3][m] * inv);
                    } else {
                        float* dst = p.rec_o + ((int64_t)rec * G + h) * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(acc[s][e][m], acc[s][e + 1][m], acc[s][e + 2][m], acc[s][e + 3][m]);
                        if (c == 0) p.rec_ml[(int64_t)rec * G + h] = make_float2(mh[s][m], lh[s][m]);
                    }
                }
            }
        }
    };

    Item ring[DEPTH];
#pragma unroll
    for (int u = 0; u < U; ++u) {   // fill the ring in stream order (the waits count on it)
        __builtin_amdgcn_sched_barrier(0);
        issue_k(u, ring[2 * u]);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(u, ring[2 * u + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int t0 = 0; t0 < ns; t0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u;
            Item& kit = ring[2 * u];
            Item& vit = ring[2 * u + 1];
            const bool live = t < ns;
            const int valid = min(16, cL - 16 * cj);   // tokens of the group (last may be short)
            float y[NSET][4];
            uint32_t pw[NSET][2];   // bf16 probabilities of tokens r + 4i, two per dword
            if (live) {
                // ---- scores of the group on the matrix cores, in log2 units
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < NQ; ++k)
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, kit.q[k]),
                            __builtin_bit_cast(bf16x8_t, qf[s][k]), sc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[s][i] = sc[i] * cl2;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue_k(t + U, kit);
            __builtin_amdgcn_sched_barrier(0);
            if (live) {
                // ---- online softmax update: lane holds tokens r + 4i of head column c
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    if (valid < 16) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) y[s][i] = (r + 4 * i < valid) ? y[s][i] : -INFINITY;
                    }
                    if constexpr (MULTI) {
                        // causal: column h (query j = h / GK) sees tokens up to L - n + j
                        const int first_q = cL - cnq;
                        if (16 * cj + 15 > first_q) {
                            const int pos = first_q + (c % G) / GK;
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                y[s][i] = (16 * cj + r + 4 * i <= pos) ? y[s][i] : -INFINITY;
                        }
                    }
                    const float mx = fmaxf(fmaxf(y[s][0], y[s][1]), fmaxf(y[s][2], y[s][3]));
                    float m_new = fmaxf(m_run[s], rows_max(mx));
                    // MULTI: a column may see no token of a segment (its query comes before
                    // the segment): 0 as the reference keeps its factors 0 instead of NaN
                    float m_ref = m_new;
                    if constexpr (MULTI) m_ref = m_new == -INFINITY ? 0.f : m_new;
                    const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_ref);
                    m_run[s] = m_new;
                    float am[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        am[m] = COLS ? col_bcast(alpha, m) : quad_bcast(alpha, m);
#pragma unroll
                    for (int e = 0; e < EV; ++e)
#pragma unroll
                        for (int m = 0; m < 4; ++m) acc[s][e][m] *= am[m];
                    // probabilities, rounded to bf16 for the matrix cores; the sum takes
                    // the rounded values too, so the weights it divides by are the ones used
                    const bf16x2_t p01 = __builtin_convertvector(
                        (f32x2_t){__builtin_amdgcn_exp2f(y[s][0] - m_ref), __builtin_amdgcn_exp2f(y[s][1] - m_ref)}, bf16x2_t);
                    const bf16x2_t p23 = __builtin_convertvector(
                        (f32x2_t){__builtin_amdgcn_exp2f(y[s][2] - m_ref), __builtin_amdgcn_exp2f(y[s][3] - m_ref)}, bf16x2_t);
                    pw[s][0] = __builtin_bit_cast(uint32_t, p01);
                    pw[s][1] = __builtin_bit_cast(uint32_t, p23);
                    l_run[s] = l_run[s] * alpha + ((lo_bf16(pw[s][0]) + hi_bf16(pw[s][0])) +
                                                   (lo_bf16(pw[s][1]) + hi_bf16(pw[s][1])));
                }
                // ---- o += p * V on the matrix cores; V rows past the end may hold anything
                if (valid < 16) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if (r + 4 * k >= valid) {
                            if constexpr (WV == 16) {
                                vit.q[k] = u32x4_t{0u, 0u, 0u, 0u};
                            } else {
                                vit.q[k >> 1][(k & 1) * 2] = 0u;
                                vit.q[k >> 1][(k & 1) * 2 + 1] = 0u;
                            }
                        }
                    }
                }
                // One v_mfma_f32_16x16x16_bf16 per output column set e: A = the lane's four
                // probabilities (row = head column c, k = tokens r + 4i, exactly as the score
                // tile left them), B = V[r + 4i][c * EV + e], gathered from the four V loads
                // with byte permutes. Output rows 4r..4r+3 repeat the G4 heads for every r.
#pragma unroll
                for (int w = 0; w < WV / 4; ++w) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                        const u32x2_t bv = {__builtin_amdgcn_perm(vword(vit, 1, w), vword(vit, 0, w), sel),
                                            __builtin_amdgcn_perm(vword(vit, 3, w), vword(vit, 2, w), sel)};
#pragma unroll
                        for (int s = 0; s < NSET; ++s) {
                            const u32x2_t av = {pw[s][0], pw[s][1]};
                            acc[s][2 * w + h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                __builtin_bit_cast(s16x4_t, av), __builtin_bit_cast(s16x4_t, bv),
                                acc[s][2 * w + h], 0, 0, 0);
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue_v(t + U, vit);
            __builtin_amdgcn_sched_barrier(0);
            if (live) {
                const bool seg_end = cj == cn - 1 || t == ns - 1;
                const int cj_next = seg_end ? 0 : cj + 1;   // defined on every path
                if (seg_end) {
                    flush();
                    if (t < ns - 1) {     // the slice goes on into the next row
                        ++cg;
                        if (cg == p.Hkv) {
                            cg = 0;
                            do {   // skip empty sequences (bounded by the batch)
                                cL = seq_len(++cb);
                            } while (cL == 0 && cb < p.B - 1);
                        }
                        cn = (cL + 15) >> 4;
                        if constexpr (MULTI) seq_queries(cb, cL, &cqs, &cnq);
                        seg_j0 = 0;
                        first_seg = false;
                        const int row = cb * p.Hkv + cg;
                        // The prefetched fragments are copied (the compiler waits for
                        // exactly their loads); fragments loaded here are waited for at
                        // once (a rare case), so that past this point the query
                        // registers hold no pending load on any path and the ring's
                        // waits stay exact.
                        if (qn_row == row) {
#pragma unroll
                            for (int s = 0; s < NSET; ++s)
#pragma unroll
                                for (int k = 0; k < NQ; ++k) qf[s][k] = qn[s][k];
                        } else {
                            load_q(row, qf);
                            __builtin_amdgcn_s_waitcnt(kWaitVm0);
                        }
                        reset();
                    }
                }
                cj = cj_next;
            }
        }
    }
}

// Merge the partial records of rows that cross slice boundaries. Workgroup w looks at the
// row holding the first group of slice w; it merges it only when that row began inside
// slice w - 1, so every split row is merged exactly once. The merge is latency-bound. A
// narrow row (G x D up to 512 floats) has its records (one per slice it touches, up to
// ~50 on the longest rows) dealt to the four waves in contiguous runs: each wave loads
// its run up to kBatch records at a time and keeps a running state, and the four states
// are combined through LDS in wave order. A wide row (G D / 4 >= 256 float4, records of
// 4 KiB or more: G = 8 decode, multi-query columns) is split by columns instead, each wave
// folding every record for its quarter of the row. The header and the descriptor are
// fetched together. The order of every sum is fixed, so results repeat bitwise.
template <int D, int G, bool MULTI>
__global__ __launch_bounds__(256) void stream_reduce_kernel(Params p) {
    constexpr int C4 = D / 4;
    constexpr int NF = G * C4;            // float4s of a row's output
    constexpr bool COLSPLIT = NF >= 256;  // wide rows: each wave takes a quarter of the columns
    constexpr int F = COLSPLIT ? NF / 256 : (NF + 63) / 64;   // float4s per lane
    constexpr int kBatch = F >= 4 ? 4 : 16 / F;   // records per round trip
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int w = blockIdx.x;
    if (w >= p.nw) return;
    const int T = p.meta[0];
    const int nwe = p.meta[1];
    const int4 d = p.desc[w];          // b, g, row start, row groups
    if (w == 0 || w >= nwe) return;
    const int s0w = (int)((int64_t)w * T / nwe);
    if (d.z >= s0w) return;            // the row starts in slice w: not split here
    const int s0p = (int)((int64_t)(w - 1) * T / nwe);
    if (d.z < s0p) return;             // began before slice w - 1: merged by an earlier group
    const int last = d.z + d.w - 1;
    const int wb = (int)(((int64_t)(last + 1) * nwe - 1) / T);   // slice holding the last group
    const int nrec = wb - w + 2;       // slices w - 1 .. wb
    const int rec_a = 2 * (w - 1) + (d.z == s0p ? 0 : 1);
    // this wave's run of records [xa, xb) and its float4s of the row, i0 + lane + 64 f
    int xa = 0, xb = nrec, i0 = 0;
    // a run that fits one batch is merged by wave 0 alone, with no exchange through LDS
    // (uniform over the workgroup: every wave reads the same descriptor)
    const bool single = !COLSPLIT && nrec <= kBatch;
    if constexpr (COLSPLIT) {
        i0 = wid * 64 * F;
    } else {
        if (single && wid != 0) return;
        const int per = single ? nrec : (nrec + 3) >> 2;
        xa = single ? 0 : min(nrec, wid * per);
        xb = min(nrec, xa + per);
    }
    int hh[F], cc[F];                  // head and float4 column of each of the lane's float4s
#pragma unroll
    for (int f = 0; f < F; ++f) {
        int i = i0 + lane + 64 * f;
        i = i < NF ? i : NF - 1;
        hh[f] = i / C4;
        cc[f] = i - hh[f] * C4;
    }
    float M[F], l[F];
    float4 o[F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
        M[f] = -INFINITY;
        l[f] = 0.f;
        o[f] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int x0 = xa; x0 < xb; x0 += kBatch) {   // running merge in slice order
        float2 ml[kBatch][F];
        float4 v[kBatch][F];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (x0 + k < xb) {         // wave-uniform: no load for a record past the run
                const int x = x0 + k;
                const int rec = x == 0 ? rec_a : 2 * (w - 1 + x);
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    ml[k][f] = p.rec_ml[(int64_t)rec * G + hh[f]];
                    v[k][f] = reinterpret_cast<const float4*>(p.rec_o + ((int64_t)rec * G + hh[f]) * D)[cc[f]];
                }
            } else {
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    ml[k][f] = make_float2(-INFINITY, 0.f);
                    v[k][f] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
#pragma unroll
        for (int f = 0; f < F; ++f) {
            float Mb = M[f];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) Mb = fmaxf(Mb, ml[k][f].x);
            // a multi-query column may see no token of a whole run: 0 as the reference
            // keeps its factors 0 instead of NaN
            const float Mr = Mb == -INFINITY ? 0.f : Mb;
            const float a = __builtin_amdgcn_exp2f(M[f] - Mr);   // 0 on the first batch
            o[f].x *= a; o[f].y *= a; o[f].z *= a; o[f].w *= a;
            l[f] *= a;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float wgt = __builtin_amdgcn_exp2f(ml[k][f].x - Mr);   // 0 past the run
                o[f].x += wgt * v[k][f].x; o[f].y += wgt * v[k][f].y;
                o[f].z += wgt * v[k][f].z; o[f].w += wgt * v[k][f].w;
                l[f] += wgt * ml[k][f].y;
            }
            M[f] = Mb;
        }
    }
    int qs = 0, n = 0;
    if constexpr (MULTI) {
        const int cap = p.max_blocks * p.bs;
        int L = p.lens[d.x];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        multi_rows(p, d.x, L, &qs, &n);
    }
    // output float4 i (head h = i / C4) of the row
    auto store = [&](int i, float4 acc, float lsum) {
        const int h = i / C4;
        const int c4 = i - h * C4;
        int64_t orow = (int64_t)d.x * p.Hq + d.y * G + h;
        if constexpr (MULTI) {
            // column h is query j = h / GK of the row's sequence (none past its query count)
            const int GK = p.Hq / p.Hkv;
            const int j = h / GK;
            if (j >= n) return;
            orow = (int64_t)(qs + j) * p.Hq + d.y * GK + (h - j * GK);
        }
        const float inv = 1.0f / lsum;
        reinterpret_cast<float4*>(p.out + orow * D)[c4] =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    };
    if (COLSPLIT || single) {
#pragma unroll
        for (int f = 0; f < F; ++f)
            if (i0 + lane + 64 * f < NF) store(i0 + lane + 64 * f, o[f], l[f]);
    } else {
        __shared__ float4 s_o[4][NF];
        __shared__ float2 s_ml[4][NF];
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int i = lane + 64 * f;
            if (i < NF) {
                s_o[wid][i] = o[f];
                s_ml[wid][i] = make_float2(M[f], l[f]);
            }
        }
        __syncthreads();
        // the four states in wave order; wave 0 holds the row's first record, whose maximum
        // is finite for every column, so Mx is finite and an empty run weighs 0
        for (int i = threadIdx.x; i < NF; i += 256) {
            float2 mlq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) mlq[q] = s_ml[q][i];
            const float Mx = fmaxf(fmaxf(mlq[0].x, mlq[1].x), fmaxf(mlq[2].x, mlq[3].x));
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            float lsum = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float wgt = __builtin_amdgcn_exp2f(mlq[q].x - Mx);
                const float4 oq = s_o[q][i];
                acc.x += wgt * oq.x; acc.y += wgt * oq.y; acc.z += wgt * oq.z; acc.w += wgt * oq.w;
                lsum += wgt * mlq[q].y;
            }
            store(i, acc, lsum);
        }
    }
}

template <bool BF16, int D, int G>
hipError_t launch_one(const Params& prm, int B, int Hkv, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if constexpr (BF16) {
        hipLaunchKernelGGL((decode_bf16_kernel<D, G, PA_BF16_DEPTH, PA_BF16_CHUNK, (PA_BF16_QLDS != 0), PA_BF16_WAVES>),
                           dim3(prm.n_parts * Hkv * B), dim3(64 * PA_BF16_WAVES), 0, s, prm);
    } else {
        const size_t lds = (size_t)prm.part_tokens * G * sizeof(float) +
                           (size_t)(prm.part_tokens / 16) * sizeof(int);
        hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G, PA_DECODE_DEPTH>),
                           dim3(prm.n_parts * Hkv * B), dim3(64), lds, s, prm);
    }
    if (prm.n_parts > 1)
        hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((prm.Hq * B + 3) / 4), dim3(256), 0, s, prm);
    return hipGetLastError();
}

// Launch shape of the stream kernel on the current device: one 4-wave workgroup per CU,
// so every SIMD runs exactly one wave (two waves sharing a SIMD are served very unevenly:
// the older one starves the younger, and equal slices then finish far apart). The
// workgroup reserves just over half of a CU's LDS, which makes that placement certain.
// Cached per device.
int stream_shape(size_t need_lds, int* nw, size_t* lds) {
    struct Entry {
        int dev, cus;
        size_t half;
    };
    static std::mutex mu;
    static Entry cache[16];
    static int used = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    Entry en{-1, 0, 0};
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].dev == dev) en = cache[i];
    }
    if (en.dev < 0) {
        int cus = 0, per_cu = 0, per_block = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return (int)e;
        e = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        if (e != hipSuccess) return (int)e;
        e = hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return (int)e;
        size_t half = (size_t)per_cu / 2 + 1024;
        if (half > (size_t)per_block) half = 0;   // cannot force it: rely on even dispatch
        en = Entry{dev, cus, half};
        std::lock_guard<std::mutex> lock(mu);
        if (used < 16) cache[used++] = en;
    }
    *nw = en.cus * 4;
    *lds = need_lds > en.half ? need_lds : en.half;
    return 0;
}

template <int D, int G, bool SPLIT, bool MULTI = false, bool DIST = false, bool FUSED = false>
hipError_t launch_stream(Params prm, int nw_req, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    size_t lds = (size_t)((FUSED ? 3 : 2) * prm.B + 1) * sizeof(int);
    int nw = 0;
    const int e = stream_shape(lds, &nw, &lds);
    if (e != 0) return (hipError_t)e;
    if (nw_req > 0) nw = nw_req;
    nw = nw > pa_internal::kMaxStreamWaves ? pa_internal::kMaxStreamWaves : nw;
    nw = (nw + 3) / 4 * 4;
    prm.nw = nw;
    hipLaunchKernelGGL((decode_stream_kernel<D, G, PA_STREAM_DEPTH, SPLIT, MULTI, DIST, FUSED>), dim3(nw / 4), dim3(256), lds, s, prm);
    hipLaunchKernelGGL((stream_reduce_kernel<D, G, MULTI>), dim3(nw), dim3(256), 0, s, prm);
    return hipGetLastError();
}

template <int D, bool SPLIT, bool FUSED>
hipError_t dispatch_stream_g(const Params& prm, int G, int nw, void* stream) {
    switch (G) {
        case 1: return launch_stream<D, 1, SPLIT, false, false, FUSED>(prm, nw, stream);
        case 2: return launch_stream<D, 2, SPLIT, false, false, FUSED>(prm, nw, stream);
        case 4: return launch_stream<D, 4, SPLIT, false, false, FUSED>(prm, nw, stream);
        case 8: return launch_stream<D, 8, SPLIT, false, (PA_STREAM_DIST8 != 0), FUSED>(prm, nw, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool FUSED>
hipError_t dispatch_stream_split(const Params& prm, int G, int nw, bool split, void* stream) {
    return split ? dispatch_stream_g<D, true, FUSED>(prm, G, nw, stream)
                 : dispatch_stream_g<D, false, FUSED>(prm, G, nw, stream);
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

int stream_waves(int32_t override_waves, int32_t* nw) {
    int n = 0;
    size_t lds = 0;
    const int e = stream_shape(0, &n, &lds);
    if (e != 0) return e;
    if (override_waves > 0) n = override_waves;
    n = n > kMaxStreamWaves ? kMaxStreamWaves : n;
    *nw = (n + 3) / 4 * 4;
    return 0;
}

int launch_decode(const DecodeLaunch& a, const char** err) {
    Params prm{};   // zero: no shared-prefix groups, no stream records
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
    prm.rec_o = a.rec_o;
    prm.rec_ml = reinterpret_cast<float2*>(a.rec_ml);
    prm.desc = reinterpret_cast<int4*>(a.desc);
    prm.meta = a.meta;
    prm.nw = 0;
    prm.min_slice = a.min_slice > 0 ? a.min_slice : 1;
    if (a.B == 0) return 0;
    const int G = a.Hq / a.Hkv;
    hipError_t e;
    if (a.path == kPathStream) {
        const bool split = a.bs < 16;
        const bool fused = a.nkey != nullptr;
        prm.nkey = static_cast<const char*>(a.nkey);
        prm.nval = static_cast<const char*>(a.nval);
        prm.nslots = a.nslots;
        if (a.D == 64)
            e = fused ? dispatch_stream_split<64, true>(prm, G, a.stream_waves, split, a.stream)
                      : dispatch_stream_split<64, false>(prm, G, a.stream_waves, split, a.stream);
        else if (a.D == 128)
            e = fused ? dispatch_stream_split<128, true>(prm, G, a.stream_waves, split, a.stream)
                      : dispatch_stream_split<128, false>(prm, G, a.stream_waves, split, a.stream);
        else
            e = hipErrorInvalidValue;
    } else {
        e = a.kv_dtype == 1 ? dispatch_d<true>(prm, a.B, a.Hkv, a.D, G, a.stream)
                            : dispatch_d<false>(prm, a.B, a.Hkv, a.D, G, a.stream);
    }
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

int launch_multi_stream(const MultiLaunch& a, const char** err) {
    Params prm{};
    prm.out = a.out;
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
    prm.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    prm.rec_o = a.rec_o;
    prm.rec_ml = reinterpret_cast<float2*>(a.rec_ml);
    prm.desc = reinterpret_cast<int4*>(a.desc);
    prm.meta = a.meta;
    prm.min_slice = a.min_slice > 0 ? a.min_slice : 1;
    prm.q_starts = a.q_starts;
    prm.total_q = a.total_q;
    prm.max_q = a.max_q;
    if (a.B == 0 || a.total_q == 0) return 0;
    hipError_t e = hipErrorInvalidValue;
    if (a.D == 64) {
        if (a.stream_g == 4) e = launch_stream<64, 4, false, true>(prm, a.stream_waves, a.stream);
        else if (a.stream_g == 8) e = launch_stream<64, 8, false, true>(prm, a.stream_waves, a.stream);
        else if (a.stream_g == 16) e = launch_stream<64, 16, false, true>(prm, a.stream_waves, a.stream);
    } else if (a.D == 128) {
        if (a.stream_g == 4) e = launch_stream<128, 4, false, true>(prm, a.stream_waves, a.stream);
        else if (a.stream_g == 8) e = launch_stream<128, 8, false, true>(prm, a.stream_waves, a.stream);
        else if (a.stream_g == 16) e = launch_stream<128, 16, false, true>(prm, a.stream_waves, a.stream);
    }
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

}  // namespace pa_internal
