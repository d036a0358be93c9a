/*
 * oracle_sanitize_driver.c -- drives every function of oracle/psq_oracle.c
 * over many small random inputs, valid and invalid, with every buffer
 * allocated at exactly the size the oracle's contract gives.  The test
 * builds it with gcc -fsanitize=address,undefined (errors abort), so an
 * out-of-bounds access, a leak or undefined behaviour anywhere in the
 * oracle fails it.  Test infrastructure only.
 *
 * usage: oracle_sanitize_driver <iterations> <seed>
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t orc_doc_segments(const int64_t *doc, int64_t B, int64_t S, int32_t *cu,
                         int32_t *max_seqlen, uint8_t *mask);
uint32_t orc_thd_tables(const int64_t *L, const int64_t *Lp, int64_t B, int64_t P, int64_t S,
                        int64_t v, int32_t *cu, int32_t *cp, int64_t *nseq, int32_t *max_seqlen,
                        int32_t *pad_between, uint8_t *mask);
void orc_copy_rows(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t row_bytes,
                   int64_t src_row_stride_bytes);
uint32_t orc_pack(const int64_t *src, int64_t src_len, const int64_t *src_off,
                  const int32_t *real_len, int64_t N, int32_t q, const int32_t *order,
                  const int64_t *pack_start, int64_t P, int32_t C, int fold, int64_t pad_token,
                  int64_t *packed, uint8_t *token_mask, int32_t *cu, int32_t *cp);
uint32_t orc_pack_rect(const int64_t *rows, int64_t W, const int32_t *real_len, int64_t N,
                       int32_t q, const int32_t *order, const int64_t *pack_start, int64_t P,
                       int32_t C, int fold, int64_t pad_token, int64_t *packed,
                       uint8_t *token_mask, int32_t *cu, int32_t *cp);
uint32_t orc_pad_mask_from_ids(const int64_t *ids, int64_t T, int64_t pad, uint8_t *mask,
                               int64_t *num_content);

static uint64_t rng_state;
/* calls that passed validation and ran the full computation */
static long ok_thd, ok_pack, ok_rect, ok_pad;

static uint64_t next_u64(void)
{
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 2685821657736338717ull;
}

/* uniform in [lo, hi] (lo when the range is empty) */
static int64_t uni(int64_t lo, int64_t hi)
{
    if (hi <= lo)
        return lo;
    return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1));
}

/* malloc of n elements of size sz; never zero bytes, so every call returns
 * a distinct block ASan can bound */
static void *alloc(int64_t n, size_t sz)
{
    void *p = malloc((size_t)(n > 0 ? n : 1) * sz);
    if (p == NULL) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void doc_case(void)
{
    int64_t B = uni(0, 5), S = uni(0, 9), T = B * S, t;
    int64_t *doc = alloc(T, sizeof(int64_t));
    int32_t *cu = alloc(T + 1, sizeof(int32_t));
    uint8_t *mask = alloc(T, 1);
    int32_t mx;
    for (t = 0; t < T; t++)
        doc[t] = uni(0, 2);
    orc_doc_segments(doc, B, S, cu, &mx, T > 0 ? mask : NULL);
    free(doc);
    free(cu);
    free(mask);
}

static void thd_case(void)
{
    const int64_t v = -1000;
    int64_t B = uni(1, 4), P = uni(0, 4), S = uni(0, 12), e;
    int64_t *L = alloc(B * P, sizeof(int64_t));
    int64_t *Lp = alloc(B * P, sizeof(int64_t));
    int32_t *cu = alloc(B * P + 1, sizeof(int32_t));
    int32_t *cp = alloc(B * P + 1, sizeof(int32_t));
    uint8_t *mask = alloc(B * S, 1);
    int64_t n;
    int32_t mx, pb;
    int with_lp = (int)uni(0, 3) != 0;
    for (e = 0; e < B * P; e++) {
        int64_t k = uni(0, 9);
        L[e] = k == 0 ? v : (k == 1 ? uni(-2, -1) : uni(0, 6));
        Lp[e] = L[e] == v ? (uni(0, 9) == 0 ? 3 : v) : L[e] + uni(-1, 3);
        if (uni(0, 19) == 0)
            Lp[e] = v;
    }
    ok_thd += orc_thd_tables(L, with_lp ? Lp : NULL, B, P, S, v, cu, cp, &n, &mx, &pb, mask) == 0;
    free(L);
    free(Lp);
    free(cu);
    free(cp);
    free(mask);
}

static void copy_case(void)
{
    int64_t rows = uni(0, 4), row_bytes = uni(0, 9), stride = row_bytes + uni(0, 3);
    int64_t src_bytes = rows > 0 ? (rows - 1) * stride + row_bytes : 0, b;
    uint8_t *src = alloc(src_bytes, 1);
    uint8_t *dst = alloc(rows * row_bytes, 1);
    for (b = 0; b < src_bytes; b++)
        src[b] = (uint8_t)uni(0, 255);
    orc_copy_rows(src, dst, rows, row_bytes, stride);
    free(src);
    free(dst);
}

static void pack_case(int rect)
{
    int64_t N = uni(0, 6), P = uni(0, 3), W = uni(0, 8), i, p;
    int32_t q = (int32_t)uni(1, 4), C = (int32_t)uni(1, 24);
    int64_t src_len = rect ? N * W : uni(0, 30);
    int64_t *src = alloc(src_len, sizeof(int64_t));
    int64_t *off = alloc(N, sizeof(int64_t));
    int32_t *rl = alloc(N, sizeof(int32_t));
    int32_t *order = alloc(N, sizeof(int32_t));
    int64_t *ps = alloc(P + 1, sizeof(int64_t));
    int64_t *packed = alloc(P * C, sizeof(int64_t));
    uint8_t *tm = alloc(P * C, 1);
    int32_t *cu = alloc(N + P, sizeof(int32_t));
    int32_t *cp = alloc(N + P, sizeof(int32_t));
    int use_order = (int)uni(0, 1);
    for (i = 0; i < src_len; i++)
        src[i] = uni(0, 1000);
    for (i = 0; i < N; i++) {
        rl[i] = (int32_t)(uni(0, 9) == 0 ? -1 : uni(0, rect ? W + 1 : 10));
        off[i] = uni(-1, src_len + 1);
        order[i] = (int32_t)(uni(0, 9) == 0 ? uni(-1, N) : uni(0, N > 0 ? N - 1 : 0));
    }
    /* pack ranges: usually a non-decreasing cover of [0, N], sometimes not */
    ps[0] = 0;
    for (p = 1; p <= P; p++)
        ps[p] = uni(0, 9) == 0 ? uni(-1, N + 1) : uni(ps[p - 1] < 0 ? 0 : ps[p - 1], N);
    if (rect)
        ok_rect += orc_pack_rect(src, W, rl, N, q, use_order ? order : NULL, ps, P, C,
                                 (int)uni(0, 1), 0, packed, tm, cu, cp) == 0;
    else
        ok_pack += orc_pack(src, src_len, off, rl, N, q, use_order ? order : NULL, ps, P, C,
                            (int)uni(0, 1), 0, packed, tm, cu, cp) == 0;
    free(src);
    free(off);
    free(rl);
    free(order);
    free(ps);
    free(packed);
    free(tm);
    free(cu);
    free(cp);
}

static void pad_case(void)
{
    int64_t T = uni(0, 10), t, nc;
    int64_t *ids = alloc(T, sizeof(int64_t));
    uint8_t *mask = alloc(T, 1);
    for (t = 0; t < T; t++)
        ids[t] = uni(0, 2);
    ok_pad += orc_pad_mask_from_ids(ids, T, uni(0, 2), mask, &nc) == 0;
    free(ids);
    free(mask);
}

int main(int argc, char **argv)
{
    long iters = argc > 1 ? atol(argv[1]) : 20000;
    long it;
    rng_state = (argc > 2 ? (uint64_t)atoll(argv[2]) : 1u) * 0x9e3779b97f4a7c15ull + 1u;
    for (it = 0; it < iters; it++) {
        doc_case();
        thd_case();
        copy_case();
        pack_case(0);
        pack_case(1);
        pad_case();
    }
    printf("ok %ld thd %ld pack %ld rect %ld pad %ld\n", iters, ok_thd, ok_pack, ok_rect, ok_pad);
    return 0;
}
