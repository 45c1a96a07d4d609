/*
 * pa_oracle.c -- the ORACLE for paged decode attention, the paged cache write and the
 * copy-on-write block clone.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load the shared object built from it. It shares no header, helper or constant with
 * the GPU path.
 *
 * It is a plain, slow, obviously correct CPU statement of what the pages define, in
 * fp64. Sources (the four web pages the method is taken from):
 *   [P1] "PagedAttention", inferensys.com glossary entry
 *   [P2] "Paged Attention" tutorial, infra.pidoku.co.in (inference engineering, vLLM, file 10)
 *   [P3] "PagedAttention: Virtual Memory for KV-Cache", insidellms.com, Chapter 4.4
 *   [P4] "PagedAttention & KV-Cache Management in High-Throughput LLM Serving",
 *        subroutine-cs.cc
 *
 * Cache layout (a reading: the pages show three layouts; this one keeps each head's
 * block as one row-major [block_size, head_dim] tile):
 *   k_cache, v_cache : [num_blocks, num_kv_heads, block_size, head_dim]
 *   block_tables     : int32 [num_seqs, max_blocks]   (logical block -> physical block)
 *   seq_lens         : int32 [num_seqs]               (tokens attended by each sequence)
 *   q                : [num_seqs, num_heads, head_dim], same element type as the cache
 * Element type 0 = fp32, 1 = bf16 (stored as its 16 raw bits).
 *
 * Parity pins (all in the CPU test suite): brute-force textbook softmax attention on
 * contiguously generated K/V, hand-worked one-token / one-block / two-token cases,
 * invariance under physical placement, prefix sharing and NaN poisoning of unused
 * slots, and byte-exact round trips of the cache write and block copy.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_BAD_TABLE = -2, ORC_DUP = -3 };

/* Decode one stored element to fp64. A bf16 value is the upper half of an fp32 word,
 * so widening its 16 bits by a left shift of 16 is exact. */
static double load_elem(const void* base, int64_t idx, int dtype) {
    if (dtype == 0) {
        return (double)((const float*)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Block-table walk for one sequence and one KV head ([P1] "Interpret Block Tables";
 * [P2] §4 PhysicalIndex and §5 "The kernel side"): token t of the sequence sits in
 * logical block t / bs, at offset t % bs inside the physical block that the table names
 * for that logical block. The gathered rows are written contiguously, in logical order,
 * into kc / vc ([L, D] each). Returns ORC_BAD_TABLE if the table names a block outside
 * the pool. */
static int materialize(double* kc, double* vc, const void* k_cache, const void* v_cache,
                       const int32_t* table, int L, int g, int Hkv, int D, int bs,
                       int num_blocks, int dtype) {
    for (int t = 0; t < L; ++t) {
        int j = t / bs;
        int off = t % bs;
        int phys = table[j];
        if (phys < 0 || phys >= num_blocks) return ORC_BAD_TABLE;
        int64_t row = (((int64_t)phys * Hkv + g) * bs + off) * (int64_t)D;
        for (int d = 0; d < D; ++d) {
            kc[(int64_t)t * D + d] = load_elem(k_cache, row + d, dtype);
            vc[(int64_t)t * D + d] = load_elem(v_cache, row + d, dtype);
        }
    }
    return ORC_OK;
}

/* Softmax attention of one query row over L contiguous K/V rows, in fp64, two passes:
 * s_t = scale * <q, k_t>; m = max_t s_t; w_t = exp(s_t - m); out = sum_t w_t v_t / sum_t w_t.
 * This is the stable softmax that [P2] §5 "The kernel side" accumulates online; both
 * give the same real number. L == 0 gives a zero row (a reading: the pages do not
 * define attention over an empty set). */
static void attend_row(double* out, const double* qrow, const double* kc, const double* vc,
                       int L, int D, double scale, double* s) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (L == 0) return;
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * kc[(int64_t)t * D + d];
        s[t] = scale * acc;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int t = 0; t < L; ++t) {
        double w = exp(s[t] - m);
        l += w;
        for (int d = 0; d < D; ++d) out[d] += w * vc[(int64_t)t * D + d];
    }
    for (int d = 0; d < D; ++d) out[d] /= l;
}

/*
 * Paged decode attention ([P1] "Interpret Block Tables" and "Handle Variable-Length
 * Sequences"; [P2] §5 "The kernel side"; [P4] §1, the decode phase).
 *
 * For each sequence b and query head h: the query head reads KV head g = h / (Hq / Hkv)
 * (consecutive query heads share a KV head); the sequence's first seq_lens[b] tokens are
 * gathered through its block table and attended with softmax(scale * q K^T) V.
 *
 * out   : fp64, [n_rows, D] if rows != NULL (row r is query row rows[r] = b * Hq + h),
 *         else [B * Hq, D].
 * scale : the fp32 value the caller passes; it is widened exactly to fp64.
 * threads <= 0 uses the OpenMP default. Work is split over (sequence, KV head) pairs;
 * each pair is computed by one thread in a fixed order, so the result does not depend
 * on the thread count.
 */
int oracle_decode(double* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* seq_lens, int B, int Hq,
                  int Hkv, int D, int bs, int num_blocks, int max_blocks, float scale,
                  int dtype, const int32_t* rows, int n_rows, int threads) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0) return ORC_BAD_ARG;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1)) return ORC_BAD_ARG;
    const int G = Hq / Hkv;
    const int all = (rows == NULL);
    const int nr = all ? B * Hq : n_rows;
    /* want[b * Hq + h] = output row index, or -1 when the row is not requested */
    int* want = (int*)malloc(sizeof(int) * (size_t)(B * Hq > 0 ? B * Hq : 1));
    if (!want) return ORC_BAD_ARG;
    for (int i = 0; i < B * Hq; ++i) want[i] = all ? i : -1;
    if (!all) {
        for (int r = 0; r < nr; ++r) {
            if (rows[r] < 0 || rows[r] >= B * Hq) { free(want); return ORC_BAD_ARG; }
            want[rows[r]] = r;
        }
    }
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0 || seq_lens[b] > max_blocks * bs) { free(want); return ORC_BAD_ARG; }
    }
    int status = ORC_OK;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int pair = 0; pair < B * Hkv; ++pair) {
        const int b = pair / Hkv;
        const int g = pair % Hkv;
        int needed = 0;
        for (int i = 0; i < G; ++i) needed |= (want[b * Hq + g * G + i] >= 0);
        if (!needed) continue;
        const int L = seq_lens[b];
        double* kc = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* vc = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* s = (double*)malloc(sizeof(double) * ((size_t)L + 1));
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        int st = (kc && vc && s && qrow) ? ORC_OK : ORC_BAD_ARG;
        if (st == ORC_OK)
            st = materialize(kc, vc, k_cache, v_cache, block_tables + (int64_t)b * max_blocks,
                             L, g, Hkv, D, bs, num_blocks, dtype);
        if (st == ORC_OK) {
            for (int i = 0; i < G; ++i) {
                const int h = g * G + i;
                const int r = want[b * Hq + h];
                if (r < 0) continue;
                for (int d = 0; d < D; ++d)
                    qrow[d] = load_elem(q, ((int64_t)b * Hq + h) * D + d, dtype);
                attend_row(out + (int64_t)r * D, qrow, kc, vc, L, D, (double)scale, s);
            }
        }
        if (st != ORC_OK) {
#pragma omp critical
            status = st;
        }
        free(kc); free(vc); free(s); free(qrow);
    }
    free(want);
    return status;
}

/*
 * Multi-query paged attention with a causal mask: several of a sequence's newest tokens
 * attend at once. This covers the prefill phase of [P4] §1 (all prompt tokens computed in
 * parallel), a later chunk of a long prompt, and several draft tokens checked in one
 * pass; the decode step of [P4] §1 is the case of one query per sequence.
 *
 * Reading (the pages give no kernel for this phase): the chunk's keys and values are
 * already in the cache (the cache write has stored them at their slots), and the chunk is
 * the sequence's last n_b tokens, n_b = q_starts[b + 1] - q_starts[b] <= seq_lens[b].
 * Query j of sequence b therefore sits at position p = seq_lens[b] - n_b + j and attends
 * to tokens 0 .. p, its own included, exactly as a decode step at length p + 1 would.
 *
 * q        : [total_q, Hq, D], total_q = q_starts[B]; the rows of sequence b are
 *            q_starts[b] .. q_starts[b + 1] - 1, in position order
 * q_starts : int32 [B + 1], q_starts[0] = 0, non-decreasing
 * out      : fp64, [n_rows, D] if rows != NULL (row r is rows[r] = qi * Hq + h for global
 *            query qi), else [total_q * Hq, D]
 * Every other argument is as for oracle_decode.
 */
int oracle_decode_multi(double* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* q_starts, int B, int Hq, int Hkv, int D, int bs,
                        int num_blocks, int max_blocks, float scale, int dtype,
                        const int32_t* rows, int n_rows, int threads) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0) return ORC_BAD_ARG;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1) || q_starts[0] != 0) return ORC_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        const int n = q_starts[b + 1] - q_starts[b];
        if (n < 0 || seq_lens[b] < n || seq_lens[b] > max_blocks * bs) return ORC_BAD_ARG;
    }
    const int G = Hq / Hkv;
    const int total = q_starts[B];
    const int all = (rows == NULL);
    const int nr = all ? total * Hq : n_rows;
    int* want = (int*)malloc(sizeof(int) * (size_t)(total * Hq > 0 ? total * Hq : 1));
    if (!want) return ORC_BAD_ARG;
    for (int i = 0; i < total * Hq; ++i) want[i] = all ? i : -1;
    if (!all) {
        for (int r = 0; r < nr; ++r) {
            if (rows[r] < 0 || rows[r] >= total * Hq) { free(want); return ORC_BAD_ARG; }
            want[rows[r]] = r;
        }
    }
    int status = ORC_OK;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int pair = 0; pair < B * Hkv; ++pair) {
        const int b = pair / Hkv;
        const int g = pair % Hkv;
        const int n = q_starts[b + 1] - q_starts[b];
        if (n == 0) continue;
        const int L = seq_lens[b];
        double* kc = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* vc = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* s = (double*)malloc(sizeof(double) * ((size_t)L + 1));
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        int st = (kc && vc && s && qrow) ? ORC_OK : ORC_BAD_ARG;
        if (st == ORC_OK)
            st = materialize(kc, vc, k_cache, v_cache, block_tables + (int64_t)b * max_blocks,
                             L, g, Hkv, D, bs, num_blocks, dtype);
        for (int j = 0; st == ORC_OK && j < n; ++j) {
            const int qi = q_starts[b] + j;
            const int p = L - n + j;           /* the query's position */
            for (int i = 0; i < G; ++i) {
                const int h = g * G + i;
                const int r = want[qi * Hq + h];
                if (r < 0) continue;
                for (int d = 0; d < D; ++d)
                    qrow[d] = load_elem(q, ((int64_t)qi * Hq + h) * D + d, dtype);
                /* the causal mask: tokens 0 .. p are the first p + 1 gathered rows */
                attend_row(out + (int64_t)r * D, qrow, kc, vc, p + 1, D, (double)scale, s);
            }
        }
        if (st != ORC_OK) {
#pragma omp critical
            status = st;
        }
        free(kc); free(vc); free(s); free(qrow);
    }
    free(want);
    return status;
}

/* Gather one sequence's contiguous K and V for one KV head (the materialize step on its
 * own, for round-trip tests): k_out, v_out are fp64 [L, D]. */
int oracle_gather(double* k_out, double* v_out, const void* k_cache, const void* v_cache,
                  const int32_t* table, int L, int g, int Hkv, int D, int bs, int num_blocks,
                  int dtype) {
    if (L < 0 || g < 0 || g >= Hkv || D <= 0 || bs <= 0) return ORC_BAD_ARG;
    return materialize(k_out, v_out, k_cache, v_cache, table, L, g, Hkv, D, bs, num_blocks,
                       dtype);
}

static int cmp_i32(const void* a, const void* b) {
    const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * Cache write: store each new token's K and V rows at its physical slot. Slot s is the
 * flat index that [P2] §4 PhysicalIndex returns, table[pos / bs] * bs + pos % bs, so the
 * row lands in block s / bs at offset s % bs. A negative slot means "no token" (padding)
 * and is skipped. The copy is of raw element bits (elt_bytes per element).
 *   key, value : [T, Hkv, D];  slot_mapping : int32 [T]
 * Duplicate non-negative slots are not a defined input: ORC_DUP.
 */
int oracle_reshape_and_cache(void* k_cache, void* v_cache, const void* key, const void* value,
                             const int32_t* slot_mapping, int T, int Hkv, int D, int bs,
                             int num_blocks, int elt_bytes) {
    if (T < 0 || Hkv <= 0 || D <= 0 || bs <= 0 || num_blocks < 0) return ORC_BAD_ARG;
    const int64_t nslots = (int64_t)num_blocks * bs;
    for (int i = 0; i < T; ++i)
        if (slot_mapping[i] >= nslots) return ORC_BAD_ARG;
    /* uniqueness of the non-negative slots: sort a copy, compare neighbours */
    int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!sorted) return ORC_BAD_ARG;
    for (int i = 0; i < T; ++i) sorted[i] = slot_mapping[i];
    qsort(sorted, (size_t)T, sizeof(int32_t), cmp_i32);
    for (int i = 1; i < T; ++i) {
        if (sorted[i] >= 0 && sorted[i] == sorted[i - 1]) { free(sorted); return ORC_DUP; }
    }
    free(sorted);
    const size_t row_bytes = (size_t)D * (size_t)elt_bytes;
    for (int i = 0; i < T; ++i) {
        const int32_t s = slot_mapping[i];
        if (s < 0) continue;
        const int64_t blk = s / bs, off = s % bs;
        for (int g = 0; g < Hkv; ++g) {
            const int64_t dst = ((blk * Hkv + g) * bs + off) * (int64_t)row_bytes;
            const int64_t src = ((int64_t)i * Hkv + g) * (int64_t)row_bytes;
            memcpy((char*)k_cache + dst, (const char*)key + src, row_bytes);
            memcpy((char*)v_cache + dst, (const char*)value + src, row_bytes);
        }
    }
    return ORC_OK;
}

/*
 * Copy-on-write block clone ([P2] §5 "Copy-on-write sharing": copy a shared block before
 * writing into it; [P4] §3): for each (src, dst) pair the whole physical block of K and of
 * V (all KV heads, all slots) is copied bit for bit. Pairs are int32 [N, 2].
 * Preconditions (ORC_DUP otherwise): destinations are distinct and no destination is
 * also a source, so the order of the copies does not matter.
 */
int oracle_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int N, int Hkv,
                       int D, int bs, int num_blocks, int elt_bytes) {
    if (N < 0 || Hkv <= 0 || D <= 0 || bs <= 0) return ORC_BAD_ARG;
    for (int i = 0; i < N; ++i) {
        const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return ORC_BAD_ARG;
        for (int k = 0; k < N; ++k) {
            if (k != i && pairs[2 * k + 1] == dst) return ORC_DUP;
            if (pairs[2 * k] == dst) return ORC_DUP;
        }
    }
    const size_t block_bytes = (size_t)Hkv * bs * D * (size_t)elt_bytes;
    for (int i = 0; i < N; ++i) {
        const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        memcpy((char*)k_cache + dst * (int64_t)block_bytes,
               (const char*)k_cache + src * (int64_t)block_bytes, block_bytes);
        memcpy((char*)v_cache + dst * (int64_t)block_bytes,
               (const char*)v_cache + src * (int64_t)block_bytes, block_bytes);
    }
    return ORC_OK;
}

/* Threads the OpenMP runtime would use by default (reported with CPU timings). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
