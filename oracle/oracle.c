/*
 * oracle.c -- plain sequential CPU oracle for the prefix-scan primitives.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source, header, table or helper with the HIP
 * library, and it includes nothing but the C standard library.
 *
 * Every function below is the plain definition of its result, written as a
 * loop in index order, in 32-bit unsigned arithmetic (C defines unsigned
 * overflow as wrap-around mod 2^32, which is the wrapping add the pages
 * require) -- and, for the u64 rows, in 64-bit unsigned arithmetic mod 2^64.  Where a page describes a schedule (the blocked three-pass scan,
 * the one-bit radix passes), that schedule is written out step by step as a
 * second function, used by the tests to check that every schedule reaches the
 * same bits as the definition.
 *
 * Sources (pages):
 *   [bend]  bendlib, "scan.bend source": header comment (contract, fork depth,
 *           three passes), "Loops (one lane)", "Pass 1", "Pass 3", "Driver",
 *           "API".
 *   [cairn] CAIRN, "Concurrency": sections "Tasks and leases", "reduce and
 *           compact" and "scan".
 *   [futh]  Futhark 0.7.4, Futhark.Pass.ExtractKernels.Segmented:
 *           regularSegmentedRedomap (Large / Small), regularSegmentedScan.
 *   [ent]   entelechy docs, package "parallel": kernel table rows
 *           compact_blank, compact_offsets, compact_gather, compact_total,
 *           sort_identity, sort_zeros, sort_place, sort_next_bit,
 *           runs_ends, runs_entries, runs_slots, the function owner, and the
 *           interface rows compact, sort, sort_pass, runs.
 *
 * Parity status: every function here is pinned by CPU tests against values
 * and properties fixed outside this file (worked examples printed on the
 * pages, closed forms, numpy library routines, brute force); none is
 * "parity unpinned".
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* O1 -- the scan, by its definition.                                        */
/* ------------------------------------------------------------------------- */

/*
 * [bend] header comment and "API": exclusive makes a[j] the sum
 * a[0] + .. + a[j-1] (a[0] becomes 0), inclusive makes a[j] the sum
 * a[0] + .. + a[j]; both return the total a[0] + .. + a[n-1]; sums wrap at
 * 2^32.  [cairn] "scan": the same two forms, and a scan may run in place
 * because each step reads only its own element.
 *
 * out may equal a (in place): each a[j] is read before out[j] is written.
 * Returns the total (0 for n == 0).
 */
uint32_t oracle_scan_u32(const uint32_t *a, uint32_t *out, uint64_t n, int inclusive)
{
    uint32_t running = 0;
    for (uint64_t j = 0; j < n; ++j) {
        uint32_t x = a[j];
        if (inclusive) {
            running += x;
            out[j] = running;
        } else {
            out[j] = running;
            running += x;
        }
    }
    return running;
}

/* ------------------------------------------------------------------------- */
/* O1c -- scan and reduce under the other integer operators.                 */
/* ------------------------------------------------------------------------- */

/*
 * [cairn] "reduce and compact": the integer operators of a reduction are
 * add_wrap, mul_wrap, &, |, ^, min and max; [cairn] "scan": a scan takes the
 * same operators, the inclusive form gives e(0) op .. op e(i), the exclusive
 * form what came before i.  Readings: values are unsigned 32-bit (min and
 * max compare them as unsigned); the exclusive output at 0, and the result
 * of an empty range, is the operator's identity (0 for add_wrap, | , ^ and
 * max; 1 for mul_wrap; 0xFFFFFFFF for & and min).  CAIRN's min and max are
 * defined on integers, signed ones included: codes 7 and 8 compare the same
 * 32-bit words as two's-complement int32 (identities INT32_MAX and
 * INT32_MIN); the other operators give the same bits either way.
 * Operator codes: 0 add_wrap, 1 mul_wrap, 2 &, 3 |, 4 ^, 5 min, 6 max,
 * 7 signed min, 8 signed max.
 */
static uint32_t op_identity(int op)
{
    switch (op) {
    case 1: return 1u;
    case 2: return 0xFFFFFFFFu;
    case 5: return 0xFFFFFFFFu;
    case 7: return 0x7FFFFFFFu;
    case 8: return 0x80000000u;
    default: return 0u;
    }
}

static uint32_t op_apply(int op, uint32_t a, uint32_t b)
{
    switch (op) {
    case 0: return a + b;
    case 1: return a * b;
    case 2: return a & b;
    case 3: return a | b;
    case 4: return a ^ b;
    case 5: return a < b ? a : b;
    case 6: return a > b ? a : b;
    case 7: return (int32_t)a < (int32_t)b ? a : b;
    case 8: return (int32_t)a > (int32_t)b ? a : b;
    default: return 0u;
    }
}

/* Returns the fold of all n values (the identity for n == 0); out may equal
 * a.  An operator code outside 0..8 returns 0 and writes nothing. */
uint32_t oracle_scan_op_u32(const uint32_t *a, uint32_t *out, uint64_t n, int op, int inclusive)
{
    if (op < 0 || op > 8)
        return 0u;
    uint32_t running = op_identity(op);
    for (uint64_t j = 0; j < n; ++j) {
        uint32_t x = a[j];
        if (inclusive) {
            running = op_apply(op, running, x);
            out[j] = running;
        } else {
            out[j] = running;
            running = op_apply(op, running, x);
        }
    }
    return running;
}

/* [cairn] "reduce and compact": the fold of n values in index order. */
uint32_t oracle_reduce_op_u32(const uint32_t *a, uint64_t n, int op)
{
    if (op < 0 || op > 8)
        return 0u;
    uint32_t acc = op_identity(op);
    for (uint64_t j = 0; j < n; ++j)
        acc = op_apply(op, acc, a[j]);
    return acc;
}

/* ------------------------------------------------------------------------- */
/* O1d -- the same scan and reduction on unsigned 64-bit values.             */
/* ------------------------------------------------------------------------- */

/*
 * [cairn] "Tasks and leases", "reduce and compact" and "scan": the page's own
 * rows are u64 (fill and total with add_wrap, the weights, the checksum's
 * mul_wrap and ^), and its pooled scan is measured on u64 elements.  The
 * operators, the operator codes and the identities are those of O1c, taken
 * mod 2^64 (C defines uint64_t overflow as wrap-around mod 2^64); the
 * identity of & and min is 2^64 - 1; signed min and max (codes 7, 8)
 * compare as int64 with identities INT64_MAX and INT64_MIN.
 */
static uint64_t op_identity64(int op)
{
    switch (op) {
    case 1: return 1u;
    case 2: return UINT64_MAX;
    case 5: return UINT64_MAX;
    case 7: return (uint64_t)INT64_MAX;
    case 8: return (uint64_t)INT64_MIN;
    default: return 0u;
    }
}

static uint64_t op_apply64(int op, uint64_t a, uint64_t b)
{
    switch (op) {
    case 0: return a + b;
    case 1: return a * b;
    case 2: return a & b;
    case 3: return a | b;
    case 4: return a ^ b;
    case 5: return a < b ? a : b;
    case 6: return a > b ? a : b;
    case 7: return (int64_t)a < (int64_t)b ? a : b;
    case 8: return (int64_t)a > (int64_t)b ? a : b;
    default: return 0u;
    }
}

/* Returns the fold of all n values (the identity for n == 0); out may equal
 * a.  An operator code outside 0..8 returns 0 and writes nothing. */
uint64_t oracle_scan_op_u64(const uint64_t *a, uint64_t *out, uint64_t n, int op, int inclusive)
{
    if (op < 0 || op > 8)
        return 0u;
    uint64_t running = op_identity64(op);
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t x = a[j];
        if (inclusive) {
            running = op_apply64(op, running, x);
            out[j] = running;
        } else {
            out[j] = running;
            running = op_apply64(op, running, x);
        }
    }
    return running;
}

/* [cairn] "reduce and compact": the fold of n u64 values in index order. */
uint64_t oracle_reduce_op_u64(const uint64_t *a, uint64_t n, int op)
{
    if (op < 0 || op > 8)
        return 0u;
    uint64_t acc = op_identity64(op);
    for (uint64_t j = 0; j < n; ++j)
        acc = op_apply64(op, acc, a[j]);
    return acc;
}

/* ------------------------------------------------------------------------- */
/* O1b -- the blocked three-pass scan of [bend], used only to check that      */
/* every fork depth gives the same bits as O1.                                */
/* ------------------------------------------------------------------------- */

/* floor(log2 n) for n >= 1. */
static unsigned floor_log2_u64(uint64_t n)
{
    unsigned lg = 0;
    while (n > 1) {
        n >>= 1;
        ++lg;
    }
    return lg;
}

/*
 * [bend] "Loops (one lane)": one lane walks entries [j, j + count) of a,
 * writing the running sum before (exclusive) or through (inclusive) each
 * entry, starting from `base`; returns the running sum past the last entry.
 */
static uint32_t one_lane_walk(uint32_t *a, uint64_t j, uint64_t count, uint32_t base, int inclusive)
{
    uint32_t s = base;
    for (uint64_t k = j; k < j + count; ++k) {
        uint32_t x = a[k];
        if (inclusive) {
            s += x;
            a[k] = s;
        } else {
            a[k] = s;
            s += x;
        }
    }
    return s;
}

/*
 * [bend] header comment ("Three passes, with no atomics") and "Driver":
 *   lg = log2 n, d = min(b, lg), e = lg - d; the array is 2^d blocks of 2^e;
 *   pass 1: s[i] = sum of block i;
 *   pass 2: s becomes its exclusive scan plus the total -- on one lane when
 *           d < 12, otherwise by this same scheme at depth floor(d/2) whose
 *           own pass 2 is always one lane (run1.sums calls run0);
 *   pass 3: block i is scanned in place from base s[i].
 * The page covers arrays of 2^lg entries only, so n must be a power of two.
 *
 * `nested_allowed` is 1 for a top-level call and 0 for the nested pass 2.
 * The 2^12 switch and the floor(d/2) depth are the page's.
 */
static uint32_t blocked_scan(uint32_t *a, uint64_t n, unsigned b, int inclusive, int nested_allowed)
{
    unsigned lg = floor_log2_u64(n);
    unsigned d = b < lg ? b : lg;
    unsigned e = lg - d;
    uint64_t blocks = (uint64_t)1 << d;
    uint64_t bsize = (uint64_t)1 << e;

    /* "Array.new(U32, d, 0)" read as 2^d zeros: one sum per block. */
    uint32_t *s = (uint32_t *)calloc((size_t)blocks, sizeof(uint32_t));
    if (!s)
        abort();

    /* Pass 1: each block's sum into s[i] (sums.leaf / sum.go). */
    for (uint64_t i = 0; i < blocks; ++i) {
        uint32_t acc = 0;
        for (uint64_t k = i * bsize; k < (i + 1) * bsize; ++k)
            acc += a[k];
        s[i] = acc;
    }

    /* Pass 2: s becomes its exclusive scan; the walk's end is the total. */
    uint32_t total;
    if (d < 12 || !nested_allowed)
        total = one_lane_walk(s, 0, blocks, 0, 0);             /* run0.sums */
    else
        total = blocked_scan(s, blocks, d / 2, 0, 0);           /* run1.sums */

    /* Pass 3: each block's scan in place from its base (puts.leaf / go). */
    for (uint64_t i = 0; i < blocks; ++i)
        (void)one_lane_walk(a, i * bsize, bsize, s[i], inclusive);

    free(s);
    return total;
}

/*
 * Returns 0 and sets *total on success; -1 when n is zero or not a power of
 * two (the page's scheme is defined on 2^lg entries only).
 */
int oracle_scan_blocked_u32(uint32_t *a, uint64_t n, unsigned b, int inclusive, uint32_t *total)
{
    if (n == 0 || (n & (n - 1)) != 0)
        return -1;
    *total = blocked_scan(a, n, b, inclusive, 1);
    return 0;
}

/*
 * The same three passes with passes 1 and 3 spread over `threads` host
 * threads, the blocks dealt out in contiguous runs; pass 2 stays one lane
 * (d < 12) or the nested scheme, exactly as in blocked_scan.  [cairn] "scan":
 * a parallel scan runs as two passes over the lane pool with a sequential
 * step between; every grouping of an integer sum gives the same bits.  Used
 * as the CPU figure beside the GPU, and checked against O1 at every depth.
 */
struct blocked_job {
    uint32_t *a;
    uint32_t *s;
    uint64_t first, last;     /* blocks [first, last) */
    uint64_t bsize;
    int inclusive;
    int pass;                 /* 1: block sums, 3: rescans */
};

static void *blocked_worker(void *arg)
{
    struct blocked_job *j = (struct blocked_job *)arg;
    for (uint64_t i = j->first; i < j->last; ++i) {
        if (j->pass == 1) {
            uint32_t acc = 0;
            for (uint64_t k = i * j->bsize; k < (i + 1) * j->bsize; ++k)
                acc += j->a[k];
            j->s[i] = acc;
        } else {
            (void)one_lane_walk(j->a, i * j->bsize, j->bsize, j->s[i], j->inclusive);
        }
    }
    return NULL;
}

/* Runs one pass over all blocks on `threads` threads; 0 on success. */
static int blocked_pass(struct blocked_job *jobs, pthread_t *tid, unsigned threads, int pass)
{
    unsigned started = 0;
    int rc = 0;
    for (unsigned t = 0; t < threads; ++t) {
        jobs[t].pass = pass;
        if (t == 0)
            continue;                       /* the calling thread runs job 0 */
        if (pthread_create(&tid[t], NULL, blocked_worker, &jobs[t]) != 0) {
            rc = -1;
            break;
        }
        started = t;
    }
    if (rc == 0)
        blocked_worker(&jobs[0]);
    for (unsigned t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    return rc;
}

/*
 * Returns 0 and sets *total on success; -1 when n is zero or not a power of
 * two, or threads is 0, or a thread cannot be started.
 */
int oracle_scan_blocked_threads_u32(uint32_t *a, uint64_t n, unsigned b, int inclusive,
                                    unsigned threads, uint32_t *total)
{
    if (n == 0 || (n & (n - 1)) != 0 || threads == 0)
        return -1;
    unsigned lg = floor_log2_u64(n);
    unsigned d = b < lg ? b : lg;
    uint64_t blocks = (uint64_t)1 << d;
    uint64_t bsize = (uint64_t)1 << (lg - d);
    if (threads > blocks)
        threads = (unsigned)blocks;
    uint32_t *s = (uint32_t *)calloc((size_t)blocks, sizeof(uint32_t));
    struct blocked_job *jobs = (struct blocked_job *)calloc(threads, sizeof(struct blocked_job));
    pthread_t *tid = (pthread_t *)calloc(threads, sizeof(pthread_t));
    if (!s || !jobs || !tid)
        abort();
    for (unsigned t = 0; t < threads; ++t) {
        jobs[t].a = a;
        jobs[t].s = s;
        jobs[t].first = blocks * t / threads;
        jobs[t].last = blocks * (t + 1) / threads;
        jobs[t].bsize = bsize;
        jobs[t].inclusive = inclusive;
    }
    int rc = blocked_pass(jobs, tid, threads, 1);
    if (rc == 0) {
        if (d < 12)
            *total = one_lane_walk(s, 0, blocks, 0, 0);
        else
            *total = blocked_scan(s, blocks, d / 2, 0, 0);
        rc = blocked_pass(jobs, tid, threads, 3);
    }
    free(tid);
    free(jobs);
    free(s);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* O2 -- segmented scan and segment sums over regular segments.              */
/* ------------------------------------------------------------------------- */

/*
 * [futh] regularSegmentedScan / regularSegmentedRedomap name a scan and a
 * reduction over regular segments: segment s is entries [s*L, s*L + L) (the
 * last one shorter when L does not divide n).  The definition:
 *   out[j]  = a[L*floor(j/L)] + .. + a[j]            (mod 2^32)
 *   sums[s] = a[s*L] + .. + a[min(s*L + L, n) - 1]   (mod 2^32)
 * The page's Large/Small strategies are schedules and do not change it.
 * out may equal a.  sums may be NULL.  Returns the number of segments
 * (ceil(n / L)), or 0 when L == 0.
 */
uint64_t oracle_segscan_u32(const uint32_t *a, uint32_t *out, uint64_t n, uint64_t L, uint32_t *sums)
{
    if (L == 0)
        return 0;
    uint32_t running = 0;
    for (uint64_t j = 0; j < n; ++j) {
        if (j % L == 0)
            running = 0;                /* a segment head restarts the sum */
        running += a[j];
        out[j] = running;
        if (sums && (j % L == L - 1 || j == n - 1))
            sums[j / L] = running;
    }
    return (n + L - 1) / L;
}

/* ------------------------------------------------------------------------- */
/* O3 -- stream compaction of flagged rows.                                  */
/* ------------------------------------------------------------------------- */

/*
 * [ent] compact: a non-zero flag keeps that element's index; the kept indices
 * are gathered to the front, and their count comes out.  The page's steps in
 * its order:
 *   compact_blank   -- every slot of the output starts at -1;
 *   compact_offsets -- inclusive prefix sum of the keep bits, so a kept
 *                      element at i belongs at offsets[i] - 1;
 *   compact_gather  -- each kept index i is written to slot offsets[i] - 1;
 *                      a zero flag writes nothing;
 *   compact_total   -- the count of kept elements (offsets[n-1], 0 if n = 0).
 * Returns the count.  out holds n entries.
 */
uint64_t oracle_compact_flags(const int32_t *flags, int32_t *out, uint64_t n)
{
    for (uint64_t k = 0; k < n; ++k)                 /* compact_blank */
        out[k] = -1;
    if (n == 0)
        return 0;

    uint64_t *offsets = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
    if (!offsets)
        abort();
    uint64_t running = 0;                            /* compact_offsets */
    for (uint64_t i = 0; i < n; ++i) {
        running += (flags[i] != 0) ? 1u : 0u;
        offsets[i] = running;
    }
    for (uint64_t i = 0; i < n; ++i)                 /* compact_gather */
        if (flags[i] != 0)
            out[offsets[i] - 1] = (int32_t)i;
    uint64_t count = offsets[n - 1];                 /* compact_total */
    free(offsets);
    return count;
}

/* ------------------------------------------------------------------------- */
/* O4 -- the stable radix-sort permutation.                                  */
/* ------------------------------------------------------------------------- */

static int cmp_u64(const void *x, const void *y)
{
    uint64_t a = *(const uint64_t *)x, b = *(const uint64_t *)y;
    return (a > b) - (a < b);
}

/*
 * The definition: perm is the permutation, in gather form (sorted[k] =
 * keys[perm[k]], as [ent] sort is read through: at(bodies, at(order, slot))),
 * that puts the keys in non-decreasing unsigned order with equal keys in
 * ascending source index -- the unique stable sorting permutation.
 * Computed by sorting the distinct 64-bit composites (key << 32 | index);
 * since no two composites are equal the order is total and stability is
 * built in.  n must be below 2^32.
 */
int oracle_stable_argsort_u32(const uint32_t *keys, int32_t *perm, uint64_t n)
{
    if (n >= ((uint64_t)1 << 32))
        return -1;
    if (n == 0)
        return 0;
    uint64_t *pairs = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
    if (!pairs)
        abort();
    for (uint64_t i = 0; i < n; ++i)
        pairs[i] = ((uint64_t)keys[i] << 32) | i;
    qsort(pairs, (size_t)n, sizeof(uint64_t), cmp_u64);
    for (uint64_t k = 0; k < n; ++k)
        perm[k] = (int32_t)(uint32_t)(pairs[k] & 0xFFFFFFFFu);
    free(pairs);
    return 0;
}

/*
 * [ent] sort / sort_pass, least significant bit first, with the pages' steps:
 *   sort_identity -- order[i] = i;
 *   per bit (sort_next_bit steps bit = 0, 1, .., 31):
 *     sort_zeros -- zeros[i] = how many places at or before i hold an element
 *                   (read through order) with a 0 at this bit;
 *     sort_place -- a zero lands at its rank among the zeros, zeros[i] - 1;
 *                   a one lands behind all Z zeros at its rank among the
 *                   ones, Z + (i + 1 - zeros[i]) - 1;
 *                   no two elements share a place.
 * Keys are full 32-bit unsigned values, so 32 one-bit passes run (the page
 * allows 1..31 bits of non-negative keys; the unsigned widening is this
 * build's reading).
 *
 * bits_per_pass == 4 runs the same loop with a 4-bit digit per pass, 8
 * passes: a stable counting pass in which a digit-d element lands at
 * (count of smaller digits) + (its rank among the digit-d elements); [cairn]
 * "scan" says the radix sort places each digit by an exclusive scan, and this
 * is that placement for 16 digit values.
 * Returns 0, or -1 for bits_per_pass other than 1 or 4 or n >= 2^31.
 */
int oracle_radix_perm_u32(const uint32_t *keys, int32_t *perm, uint64_t n, int bits_per_pass)
{
    if ((bits_per_pass != 1 && bits_per_pass != 4) || n >= ((uint64_t)1 << 31))
        return -1;
    if (n == 0)
        return 0;
    uint32_t *order = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
    uint32_t *next = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
    uint32_t *zeros = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
    if (!order || !next || !zeros)
        abort();

    for (uint64_t i = 0; i < n; ++i)                 /* sort_identity */
        order[i] = (uint32_t)i;

    if (bits_per_pass == 1) {
        for (unsigned bit = 0; bit < 32; ++bit) {    /* sort_next_bit */
            uint32_t z = 0;                          /* sort_zeros */
            for (uint64_t i = 0; i < n; ++i) {
                if (((keys[order[i]] >> bit) & 1u) == 0)
                    ++z;
                zeros[i] = z;
            }
            uint32_t Z = z;
            for (uint64_t i = 0; i < n; ++i) {       /* sort_place */
                uint64_t dest;
                if (((keys[order[i]] >> bit) & 1u) == 0)
                    dest = (uint64_t)zeros[i] - 1;
                else
                    dest = (uint64_t)Z + (i + 1 - zeros[i]) - 1;
                next[dest] = order[i];
            }
            uint32_t *t = order;
            order = next;
            next = t;
        }
    } else {
        for (unsigned shift = 0; shift < 32; shift += 4) {
            uint64_t count[16] = {0};
            for (uint64_t i = 0; i < n; ++i)
                ++count[(keys[order[i]] >> shift) & 15u];
            uint64_t base[16];
            uint64_t acc = 0;                        /* exclusive scan of counts */
            for (int dgt = 0; dgt < 16; ++dgt) {
                base[dgt] = acc;
                acc += count[dgt];
            }
            for (uint64_t i = 0; i < n; ++i) {       /* stable placement */
                unsigned dgt = (keys[order[i]] >> shift) & 15u;
                next[base[dgt]++] = order[i];
            }
            uint32_t *t = order;
            order = next;
            next = t;
        }
    }

    for (uint64_t k = 0; k < n; ++k)
        perm[k] = (int32_t)order[k];
    free(order);
    free(next);
    free(zeros);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O5 -- runs: entries laid out by owner.                                     */
/* ------------------------------------------------------------------------- */

/*
 * [ent] runs_ends: the end of every owner's run, the counts' inclusive
 * prefix sums; owner i then holds slots ends[i] - counts[i] .. ends[i] - 1.
 * [ent] runs_entries: the number of entries, never below one, so the row of
 * slots always exists.
 * Readings: counts are unsigned 32-bit and the sums wrap at 2^32 as the scan's
 * do; for n == 0 the runs hold nothing and entries is 1.
 * Writes ends[0..n) and returns entries = max(ends[n-1], 1).
 */
uint32_t oracle_runs_u32(const uint32_t *counts, uint32_t *ends, uint64_t n)
{
    uint32_t running = 0;
    for (uint64_t i = 0; i < n; ++i) {
        running += counts[i];
        ends[i] = running;
    }
    return running > 1u ? running : 1u;
}

/* [ent] runs_slots: the row the runs are laid in, every slot -1. */
void oracle_runs_slots(int32_t *slots, uint64_t entries)
{
    for (uint64_t k = 0; k < entries; ++k)
        slots[k] = -1;
}

/*
 * Every entry's owner, by the scatter [ent] "runs" describes: a walk over
 * the owners in order in which owner i emits its counts[i] entries at
 * ends[i] - counts[i] plus their rank.  `owner` has room for `total` entries
 * (the sum of the counts, which must not wrap); returns 0, or -1 if the
 * counts do not sum to `total`.
 */
int oracle_runs_owner_all(const uint32_t *counts, uint64_t n, int32_t *owner, uint64_t total)
{
    uint64_t at = 0;
    for (uint64_t i = 0; i < n; ++i) {
        for (uint32_t r = 0; r < counts[i]; ++r) {
            if (at >= total)
                return -1;
            owner[at++] = (int32_t)i;
        }
    }
    return at == total ? 0 : -1;
}

/*
 * [ent] owner(e, ends): the owner whose run holds entry e -- the least i
 * with ends[i] > e, since runs [ends[i] - counts[i], ends[i]) follow one
 * another in order and an empty run holds nothing.  Reading: an entry no
 * run holds (e >= ends[n-1]) has owner -1, the page's "nothing" value.
 * Walks the ends one by one (no search).
 */
int32_t oracle_runs_owner(const uint32_t *ends, uint64_t n, uint32_t e)
{
    for (uint64_t i = 0; i < n; ++i)
        if (ends[i] > e)
            return (int32_t)i;
    return -1;
}

/* ------------------------------------------------------------------------- */
/* O2b -- segmented scan over irregular segments given by head flags.         */
/* ------------------------------------------------------------------------- */

/*
 * [futh] names a segmented scan over regular segments only; here segments
 * are irregular: element j starts a segment when j == 0 or flags[j] != 0
 * (reading: element 0 always starts one, whatever flags[0] holds).
 * out[j] = a[h] + .. + a[j] (mod 2^32) with h the last start at or before j;
 * sums[s], when sums is not NULL, is the total of segment s (segments
 * numbered from 0 in order).  out may equal a.  Returns the number of
 * segments (0 for n == 0).
 */
uint64_t oracle_segscan_flags_u32(const uint32_t *a, const uint32_t *flags, uint32_t *out,
                                  uint64_t n, uint32_t *sums)
{
    uint32_t running = 0;
    uint64_t segs = 0;
    for (uint64_t j = 0; j < n; ++j) {
        if (j == 0 || flags[j] != 0) {
            running = 0;
            ++segs;
        }
        running += a[j];
        out[j] = running;
        if (sums)
            sums[segs - 1] = running;
    }
    return segs;
}
