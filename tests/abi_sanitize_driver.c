/*
 * abi_sanitize_driver.c -- drives the host side of the psq C ABI (argument
 * validation, workspace sizing, grid and copy planning, launch set-up) on a
 * CPU, with the HIP runtime replaced by abi_sanitize_stubs.c.  The test builds
 * the library's sources host-only with -fsanitize=address,undefined (errors
 * abort), so signed overflow in the size arithmetic, an out-of-bounds access
 * or a leak anywhere in that code fails it.  Device pointers are never
 * dereferenced by the host code, so fake addresses stand in for them.
 * Test infrastructure only.
 *
 * It runs, in order:
 *  1. every validation case of tests/test_abi_host.py;
 *  2. a seeded fuzz of every entry point, sizes drawn around the int32 and
 *     int64 limits, strides and copies drawn to overlap, num_chunks around
 *     its edges, pointers null, aligned and misaligned;
 *  3. with each fuzzed size, consistency of the workspace queries: a query of
 *     0 means the call rejects the sizes; a call that succeeds with the
 *     queried bytes fails with one byte less.
 * A call that succeeds must have launched kernels of legal shape (the stub
 * aborts otherwise).
 *
 * usage: abi_sanitize_driver <iterations> <seed>
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "psq.h"

extern long stub_launches;

#define FAKE ((uintptr_t)0x10000)
#define P(x) ((void *)(uintptr_t)(x))

static long failures, checks;

static void expect(int line, int got, int want)
{
    ++checks;
    if (got != want) {
        fprintf(stderr, "line %d: got %d, want %d\n", line, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect(__LINE__, (call), (want))

/* ------------------------------------------------------------------------ */
/* argument bundles with the defaults of tests/test_abi_host.py              */
/* ------------------------------------------------------------------------ */
typedef struct {
    const void *doc; int dt; int64_t B, S; void *cu, *n, *mx, *mask, *st, *ws; size_t wsb;
} DocA;
static DocA doc_defaults(void)
{
    DocA a = {P(FAKE), PSQ_I32, 4, 64, P(FAKE), P(FAKE), P(FAKE), NULL, NULL, NULL, 0};
    return a;
}
static int doc_call(DocA a)
{
    return psq_params_from_doc_ids(a.doc, a.dt, a.B, a.S, (int32_t *)a.cu, (int32_t *)a.n,
                                   (int32_t *)a.mx, (uint8_t *)a.mask, (int32_t *)a.st, a.ws,
                                   a.wsb, NULL);
}
static int noalloc_call(DocA a)
{
    return psq_params_from_doc_ids_noalloc(a.doc, a.dt, a.B, a.S, (int32_t *)a.cu,
                                           (int32_t *)a.n, (int32_t *)a.mx, (uint8_t *)a.mask,
                                           (int32_t *)a.st, NULL);
}

static psq_thd_layout layout(int kind, const void *L, const void *Lp, int dt, int64_t P_,
                             int64_t pad, const void *doc, int doc_dt)
{
    psq_thd_layout l;
    memset(&l, 0, sizeof l);
    l.kind = kind;
    l.seq_lens = L;
    l.seq_lens_padded = Lp;
    l.lens_dtype = dt;
    l.P = P_;
    l.pad_value = pad;
    l.doc_ids = doc;
    l.doc_dtype = doc_dt;
    return l;
}
static psq_thd_layout lens_layout(const void *L, const void *Lp, int dt, int64_t P_)
{
    return layout(PSQ_LAYOUT_SEQ_LENS, L, Lp, dt, P_, -1000, NULL, PSQ_I32);
}
static psq_thd_layout doc_layout(const void *doc, int doc_dt)
{
    return layout(PSQ_LAYOUT_DOC_IDS, NULL, NULL, PSQ_I64, 0, -1000, doc, doc_dt);
}

typedef struct {
    const psq_thd_layout *lay; int64_t B, S; void *cu, *cp, *n, *mx, *pb, *mask;
    const psq_copy *copies; int n_copies; void *st, *ws; size_t wsb;
} ThdA;
static ThdA thd_defaults(const psq_thd_layout *lay)
{
    ThdA a = {lay, 2, 6, P(FAKE), NULL, P(FAKE), P(FAKE), P(FAKE), NULL, NULL, 0, P(FAKE),
              P(FAKE), 0};
    return a;
}
static int thd_call(ThdA a)
{
    return psq_process_thd(a.lay, a.B, a.S, (int32_t *)a.cu, (int32_t *)a.cp, (int32_t *)a.n,
                           (int32_t *)a.mx, (int32_t *)a.pb, (uint8_t *)a.mask, a.copies,
                           a.n_copies, (int32_t *)a.st, a.ws, a.wsb, NULL);
}

typedef struct {
    const psq_thd_layout *lay; int64_t B, S, G; void *cu, *cp, *w, *n, *mx, *pb, *mask, *st, *ws;
    size_t wsb;
} SplitA;
static SplitA split_defaults(const psq_thd_layout *lay)
{
    SplitA a = {lay, 4, 6, 2, P(FAKE), NULL, P(FAKE), P(FAKE), P(FAKE), P(FAKE), NULL, P(FAKE),
                P(FAKE), (size_t)1 << 20};
    return a;
}
static int split_call(SplitA a)
{
    return psq_split_thd(a.lay, a.B, a.S, a.G, (int32_t *)a.cu, (int32_t *)a.cp, (int32_t *)a.w,
                         (int32_t *)a.n, (int32_t *)a.mx, (int32_t *)a.pb, (uint8_t *)a.mask,
                         NULL, 0, (int32_t *)a.st, a.ws, a.wsb, NULL);
}

typedef struct {
    const void *ids; int dt; int64_t T, pad; void *mask, *nc, *st, *ws; size_t wsb;
} PadA;
static PadA pad_defaults(void)
{
    PadA a = {P(FAKE), PSQ_I64, 64, 0, P(FAKE), NULL, P(FAKE), P(FAKE), 256};
    return a;
}
static int pad_call(PadA a)
{
    return psq_padding_mask_from_token_ids(a.ids, a.dt, a.T, a.pad, (uint8_t *)a.mask,
                                           (int32_t *)a.nc, (int32_t *)a.st, a.ws, a.wsb, NULL);
}

typedef struct {
    const void *src; int64_t src_len; const void *off, *rl; int64_t N; int32_t q;
    const void *order, *ps; int64_t P_; int32_t C; int fold; int64_t pad;
    void *packed, *tm, *cu, *cp, *st, *ws; size_t wsb;
} PackA;
static PackA pack_defaults(void)
{
    PackA a = {P(FAKE), 100, P(FAKE), P(FAKE), 4, 4, NULL, P(FAKE), 2, 36, 1, 0, P(FAKE),
               P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 256};
    return a;
}
static int pack_call(PackA a)
{
    return psq_pack_rows((const int64_t *)a.src, a.src_len, (const int64_t *)a.off,
                         (const int32_t *)a.rl, a.N, a.q, (const int32_t *)a.order,
                         (const int64_t *)a.ps, a.P_, a.C, a.fold, a.pad, (int64_t *)a.packed,
                         (uint8_t *)a.tm, (int32_t *)a.cu, (int32_t *)a.cp, (int32_t *)a.st,
                         a.ws, a.wsb, NULL);
}

typedef struct {
    const void *rows; int64_t W; const void *rl; int64_t N; int32_t q; const void *order, *ps;
    int64_t P_; int32_t C; int fold; int64_t pad; void *packed, *tm, *cu, *cp, *st, *ws;
    size_t wsb;
} RectA;
static RectA rect_defaults(void)
{
    RectA a = {P(FAKE), 10, P(FAKE), 2, 4, NULL, P(FAKE), 1, 20, 0, 0, P(FAKE), P(FAKE),
               P(FAKE), P(FAKE), P(FAKE), P(FAKE), 256};
    return a;
}
static int rect_call(RectA a)
{
    return psq_pack_padded_rows((const int64_t *)a.rows, a.W, (const int32_t *)a.rl, a.N, a.q,
                                (const int32_t *)a.order, (const int64_t *)a.ps, a.P_, a.C,
                                a.fold, a.pad, (int64_t *)a.packed, (uint8_t *)a.tm,
                                (int32_t *)a.cu, (int32_t *)a.cp, (int32_t *)a.st, a.ws, a.wsb,
                                NULL);
}

static psq_copy copy_of(uintptr_t src, uintptr_t dst, int64_t rows, int64_t row_bytes,
                        int64_t src_stride, int64_t dst_stride)
{
    psq_copy c = {P(src), P(dst), rows, row_bytes, src_stride, dst_stride};
    return c;
}

/* ------------------------------------------------------------------------ */
/* 1. the cases of tests/test_abi_host.py                                    */
/* ------------------------------------------------------------------------ */
static void host_test_cases(void)
{
    int i;
    const int64_t I31 = (int64_t)1 << 31;

    /* test_status_strings */
    if (strcmp(psq_status_string(0, 0), "ok") != 0 ||
        strcmp(psq_status_string(999, 0), "unknown error code") != 0 ||
        !strstr(psq_status_string(PSQ_ERR_WORKSPACE, 0), "workspace") ||
        !strstr(psq_status_string(PSQ_DATA_PACK_OVERFLOW, 1), "capacity") ||
        !strstr(psq_status_string(PSQ_DATA_EMPTY_ROW, 1), "no sequence") ||
        !strstr(psq_status_string(PSQ_DATA_PAD_IS_CONTENT, 1), "content")) {
        fprintf(stderr, "status strings\n");
        ++failures;
    }

    /* test_workspace_sizes */
    {
        psq_thd_layout lay = lens_layout(P(FAKE), NULL, PSQ_I64, 64);
        psq_thd_layout huge = lens_layout(P(FAKE), NULL, PSQ_I64, (int64_t)1 << 40);
        psq_thd_layout bad = layout(7, NULL, NULL, PSQ_I64, 0, -1000, NULL, PSQ_I32);
        psq_thd_layout doc = doc_layout(P(FAKE), PSQ_I32);
        size_t a = psq_params_from_doc_ids_workspace(4, 64);
        size_t b = psq_params_from_doc_ids_workspace(32, 32768);
        size_t one = psq_split_thd_workspace(&lay, 16, 8192, 1);
        size_t four = psq_split_thd_workspace(&lay, 16, 8192, 4);
        EXPECT(psq_params_from_doc_ids_workspace(0, 0) >= 256, 1);
        EXPECT(a >= 256 && b > a && b % 256 == 0, 1);
        EXPECT(psq_process_thd_workspace(&lay, 16, 8192) >= 256 + 8 * 16, 1);
        EXPECT(psq_pack_rows_workspace(65536, 3555, 16384) >= 256, 1);
        EXPECT(psq_padding_mask_from_token_ids_workspace(131072) >= 256, 1);
        EXPECT(one == psq_process_thd_workspace(&lay, 16, 8192), 1);
        EXPECT(four >= one + 2 * 4 * 4 * (4 * 64 + 1), 1);
        EXPECT((int)psq_split_thd_workspace(&lay, 16, 8192, 3), 0);
        EXPECT((int)psq_split_thd_workspace(&lay, 16, 8192, 0), 0);
        EXPECT((int)psq_params_from_doc_ids_workspace((int64_t)1 << 40, (int64_t)1 << 40), 0);
        EXPECT((int)psq_params_from_doc_ids_workspace((int64_t)1 << 16, (int64_t)1 << 15), 0);
        EXPECT(psq_params_from_doc_ids_workspace(((int64_t)1 << 16) - 1, (int64_t)1 << 15) > 0, 1);
        EXPECT((int)psq_process_thd_workspace(&lay, (int64_t)1 << 40, (int64_t)1 << 40), 0);
        EXPECT((int)psq_process_thd_workspace(&huge, (int64_t)1 << 40, 0), 0);
        EXPECT((int)psq_split_thd_workspace(&huge, (int64_t)1 << 40, 0, 1), 0);
        EXPECT((int)psq_split_thd_workspace(&lay, (int64_t)1 << 32, 0, (int64_t)1 << 32), 0);
        EXPECT((int)psq_process_thd_workspace(&bad, 4, 4), 0);
        EXPECT(psq_process_thd_workspace(&doc, 4, 64) == a, 1);
    }

    /* test_doc_ids_validation */
    {
        DocA a;
        a = doc_defaults(); a.B = -1; EXPECT(doc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.S = -3; EXPECT(doc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.dt = 7; EXPECT(doc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.B = 1 << 16; a.S = 1 << 15; EXPECT(doc_call(a), PSQ_ERR_OVERFLOW);
        a = doc_defaults(); a.B = 1; a.S = I31; EXPECT(doc_call(a), PSQ_ERR_OVERFLOW);
        a = doc_defaults(); a.cu = NULL; EXPECT(doc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.doc = NULL; EXPECT(doc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.ws = NULL; EXPECT(doc_call(a), PSQ_ERR_WORKSPACE);
        a = doc_defaults(); a.ws = P(FAKE); a.wsb = 8; EXPECT(doc_call(a), PSQ_ERR_WORKSPACE);
    }

    /* test_doc_ids_noalloc_validation */
    {
        DocA a;
        a = doc_defaults(); a.B = -1; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.S = -3; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.dt = 7; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.B = 1 << 16; a.S = 1 << 15; EXPECT(noalloc_call(a), PSQ_ERR_OVERFLOW);
        a = doc_defaults(); a.B = 1; a.S = I31; EXPECT(noalloc_call(a), PSQ_ERR_OVERFLOW);
        a = doc_defaults(); a.cu = NULL; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.n = NULL; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.mx = NULL; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
        a = doc_defaults(); a.doc = NULL; EXPECT(noalloc_call(a), PSQ_ERR_ARG);
    }

    /* test_workspace_alignment */
    for (i = 4; i <= 12; i += 4) {
        psq_thd_layout lay = lens_layout(P(FAKE), P(FAKE), PSQ_I64, 2);
        psq_thd_layout doc = doc_layout(P(FAKE), PSQ_I32);
        DocA d = doc_defaults();
        PadA pa = pad_defaults();
        PackA pk = pack_defaults();
        RectA r = rect_defaults();
        ThdA t = thd_defaults(&lay);
        ThdA td = thd_defaults(&doc);
        SplitA s = split_defaults(&lay);
        d.ws = P(FAKE + i); d.wsb = (size_t)1 << 20; EXPECT(doc_call(d), PSQ_ERR_WORKSPACE);
        pa.ws = P(FAKE + i); EXPECT(pad_call(pa), PSQ_ERR_WORKSPACE);
        pk.ws = P(FAKE + i); EXPECT(pack_call(pk), PSQ_ERR_WORKSPACE);
        r.ws = P(FAKE + i); EXPECT(rect_call(r), PSQ_ERR_WORKSPACE);
        t.ws = P(FAKE + i); t.wsb = (size_t)1 << 20; EXPECT(thd_call(t), PSQ_ERR_WORKSPACE);
        td.ws = P(FAKE + i); td.wsb = (size_t)1 << 20; EXPECT(thd_call(td), PSQ_ERR_WORKSPACE);
        s.ws = P(FAKE + i); s.wsb = (size_t)1 << 20; EXPECT(split_call(s), PSQ_ERR_WORKSPACE);
    }

    /* test_process_thd_validation */
    {
        psq_thd_layout lay = lens_layout(P(FAKE), P(FAKE), PSQ_I64, 2);
        psq_thd_layout l5 = layout(5, NULL, NULL, PSQ_I64, 0, -1000, NULL, PSQ_I32);
        psq_thd_layout l9 = lens_layout(P(FAKE), NULL, 9, 2);
        psq_thd_layout lneg = lens_layout(P(FAKE), NULL, PSQ_I64, -1);
        psq_thd_layout lnull = lens_layout(NULL, NULL, PSQ_I64, 2);
        psq_thd_layout d3 = doc_layout(P(FAKE), 3);
        psq_thd_layout dnull = doc_layout(NULL, PSQ_I32);
        psq_thd_layout big = lens_layout(P(FAKE), NULL, PSQ_I64, (int64_t)1 << 20);
        psq_thd_layout huge = lens_layout(P(FAKE), NULL, PSQ_I64, (int64_t)1 << 40);
        psq_copy c[9];
        ThdA a;
        a = thd_defaults(NULL); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&lay); a.B = -1; EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&lay); a.st = NULL; EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&lay); a.cu = NULL; EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&l5); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&l9); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&lneg); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&lnull); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&d3); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&dnull); EXPECT(thd_call(a), PSQ_ERR_ARG);
        a = thd_defaults(&big); a.B = 1 << 11; a.S = 4; EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        a = thd_defaults(&lay); a.B = 1 << 20; a.S = 1 << 12; EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        a = thd_defaults(&huge); a.B = (int64_t)1 << 40; a.S = 0;
        EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        a = thd_defaults(&lay); EXPECT(thd_call(a), PSQ_ERR_WORKSPACE);
        a = thd_defaults(&lay); a.ws = NULL; a.wsb = (size_t)1 << 20;
        EXPECT(thd_call(a), PSQ_ERR_WORKSPACE);
        for (i = 0; i < 9; ++i) c[i] = copy_of(FAKE, FAKE + 4096, 1, 64, 64, 0);
        a = thd_defaults(&lay); a.copies = c; a.n_copies = 9; a.wsb = (size_t)1 << 20;
        EXPECT(thd_call(a), PSQ_ERR_ARG);
        a.n_copies = 1;
        c[0] = copy_of(0, FAKE, 1, 64, 64, 0); EXPECT(thd_call(a), PSQ_ERR_ARG);
        c[0] = copy_of(FAKE, FAKE + 32, 1, 64, 64, 0); EXPECT(thd_call(a), PSQ_ERR_ARG);
        c[0] = copy_of(FAKE, FAKE + 65536, 4, 64, 32, 0); EXPECT(thd_call(a), PSQ_ERR_ARG);
        c[0] = copy_of(FAKE, FAKE + 65536, -1, 64, 64, 0); EXPECT(thd_call(a), PSQ_ERR_ARG);
        c[0] = copy_of(FAKE, FAKE + 65536, 4, 64, 64, 32); EXPECT(thd_call(a), PSQ_ERR_ARG);
        c[0] = copy_of(FAKE, FAKE + 65536, 1, 64, 64, -8); EXPECT(thd_call(a), PSQ_ERR_ARG);
        c[0] = copy_of(FAKE + 1, FAKE + ((uintptr_t)1 << 40), 1, I31 + 1, I31 + 1, 0);
        EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        c[0] = copy_of(FAKE, FAKE + ((uintptr_t)1 << 40), (int64_t)1 << 40, 1 << 30, 1 << 30, 0);
        EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        a = thd_defaults(&lay); a.B = 1 << 24; a.S = 64; EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        a = thd_defaults(&lay); a.B = (1 << 24) - 1; a.S = 64; EXPECT(thd_call(a), PSQ_ERR_WORKSPACE);
        c[0] = copy_of(FAKE, FAKE + ((uintptr_t)1 << 40), 1, (int64_t)1 << 34, (int64_t)1 << 34, 0);
        a = thd_defaults(&lay); a.B = 3 << 22; a.S = 64; a.copies = c; a.n_copies = 1;
        EXPECT(thd_call(a), PSQ_ERR_OVERFLOW);
        a.B = (3 << 22) - 1; EXPECT(thd_call(a), PSQ_ERR_WORKSPACE);
        c[0] = copy_of(FAKE + 4096, FAKE, 4, 64, 64, 2048);
        a = thd_defaults(&lay); a.copies = c; a.n_copies = 1; a.wsb = (size_t)1 << 20;
        EXPECT(thd_call(a), PSQ_ERR_ARG);
    }

    /* test_split_thd_validation */
    {
        psq_thd_layout lay = lens_layout(P(FAKE), P(FAKE), PSQ_I64, 1);
        psq_thd_layout doc = doc_layout(P(FAKE), PSQ_I32);
        psq_thd_layout wide = layout(PSQ_LAYOUT_SEQ_LENS, P(FAKE), P(FAKE), PSQ_I64, 1,
                                     -((int64_t)1 << 40), NULL, PSQ_I32);
        psq_thd_layout huge = lens_layout(P(FAKE), P(FAKE), PSQ_I64, (int64_t)1 << 40);
        SplitA a;
        a = split_defaults(NULL); EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&lay); a.G = 0; EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&lay); a.G = 3; EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&doc); EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&lay); a.w = NULL; EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&wide); EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&lay); a.n = NULL; EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&lay); a.st = NULL; EXPECT(split_call(a), PSQ_ERR_ARG);
        a = split_defaults(&lay); a.B = 1 << 20; a.S = 1 << 12; a.G = 1 << 10;
        EXPECT(split_call(a), PSQ_ERR_OVERFLOW);
        a = split_defaults(&huge); a.B = (int64_t)1 << 40; a.S = 0; a.G = 1;
        EXPECT(split_call(a), PSQ_ERR_OVERFLOW);
        a = split_defaults(&lay); a.B = (int64_t)1 << 40; a.S = 0; a.G = (int64_t)1 << 40;
        EXPECT(split_call(a), PSQ_ERR_OVERFLOW);
        a = split_defaults(&lay); a.B = (int64_t)1 << 32; a.S = 0; a.G = (int64_t)1 << 32;
        EXPECT(split_call(a), PSQ_ERR_OVERFLOW);
        a = split_defaults(&lay); a.B = 1 << 24; a.S = 64; a.G = 1 << 10;
        EXPECT(split_call(a), PSQ_ERR_OVERFLOW);
        a = split_defaults(&lay); a.B = (1 << 24) - 1024; a.S = 64; a.G = 1 << 10; a.ws = NULL;
        EXPECT(split_call(a), PSQ_ERR_WORKSPACE);
        a = split_defaults(&lay); a.ws = NULL; EXPECT(split_call(a), PSQ_ERR_WORKSPACE);
        a = split_defaults(&lay); a.wsb = 256; EXPECT(split_call(a), PSQ_ERR_WORKSPACE);
    }

    /* test_padding_mask_from_token_ids_validation */
    {
        PadA a;
        a = pad_defaults(); a.T = -1; EXPECT(pad_call(a), PSQ_ERR_ARG);
        a = pad_defaults(); a.dt = 2; EXPECT(pad_call(a), PSQ_ERR_ARG);
        a = pad_defaults(); a.T = I31; EXPECT(pad_call(a), PSQ_ERR_OVERFLOW);
        a = pad_defaults(); a.ids = NULL; EXPECT(pad_call(a), PSQ_ERR_ARG);
        a = pad_defaults(); a.mask = NULL; EXPECT(pad_call(a), PSQ_ERR_ARG);
        a = pad_defaults(); a.st = NULL; EXPECT(pad_call(a), PSQ_ERR_ARG);
        a = pad_defaults(); a.ws = NULL; EXPECT(pad_call(a), PSQ_ERR_WORKSPACE);
        a = pad_defaults(); a.wsb = 8; EXPECT(pad_call(a), PSQ_ERR_WORKSPACE);
    }

    /* test_pack_padded_rows_validation */
    {
        RectA a;
        a = rect_defaults(); a.W = -1; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.q = 0; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.C = 0; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.N = 1 << 30; a.W = (int64_t)1 << 33;
        EXPECT(rect_call(a), PSQ_ERR_OVERFLOW);
        a = rect_defaults(); a.rows = NULL; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.rl = NULL; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.ps = NULL; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.cu = NULL; EXPECT(rect_call(a), PSQ_ERR_ARG);
        a = rect_defaults(); a.ws = NULL; EXPECT(rect_call(a), PSQ_ERR_WORKSPACE);
    }

    /* test_pack_rows_validation */
    {
        PackA a;
        a = pack_defaults(); a.q = 0; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.C = 0; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.C = (1 << 30) + 1; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.N = -1; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.P_ = -1; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.N = I31 - 5; a.P_ = 10; EXPECT(pack_call(a), PSQ_ERR_OVERFLOW);
        a = pack_defaults(); a.ps = NULL; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.st = NULL; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.packed = NULL; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.rl = NULL; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.src = NULL; EXPECT(pack_call(a), PSQ_ERR_ARG);
        a = pack_defaults(); a.ws = NULL; EXPECT(pack_call(a), PSQ_ERR_WORKSPACE);
        a = pack_defaults(); a.wsb = 16; EXPECT(pack_call(a), PSQ_ERR_WORKSPACE);
        a = pack_defaults(); a.P_ = 1 << 26; a.C = 64; a.ws = NULL;
        EXPECT(pack_call(a), PSQ_ERR_OVERFLOW);
        a = pack_defaults(); a.P_ = (1 << 26) - 1; a.C = 64; a.ws = NULL;
        EXPECT(pack_call(a), PSQ_ERR_WORKSPACE);
        a = pack_defaults(); a.P_ = 1 << 22; a.C = 16384; a.ws = NULL;
        EXPECT(pack_call(a), PSQ_ERR_OVERFLOW);
        a = pack_defaults(); a.P_ = 1 << 21; a.C = 16384; a.ws = NULL;
        EXPECT(pack_call(a), PSQ_ERR_WORKSPACE);
    }
}

/* ------------------------------------------------------------------------ */
/* 2./3. seeded fuzz                                                         */
/* ------------------------------------------------------------------------ */
static uint64_t rng_state;

static uint64_t next_u64(void)
{
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u64() % (uint64_t)n) : 0; }

/* a size from an edge-heavy mixture: small values, the int32 and int64
 * limits and their neighbours, powers of two, negatives */
static int64_t edge_size(void)
{
    static const int64_t edges[] = {0, 1, 2, 3, 4, 7, 8, 63, 64, 65, 255, 256, 896, 1023, 1024,
                                    4095, 4096, 4097, 65535, 65536, 1 << 20, (1 << 24) - 1,
                                    1 << 24, 1 << 26, (1 << 30) - 1, 1 << 30, (1 << 30) + 1,
                                    0x7fffffffLL - 1, 0x7fffffffLL, 0x80000000LL,
                                    0x100000000LL, 1LL << 40, 1LL << 62, INT64_MAX - 1,
                                    INT64_MAX, -1, -2, -1000, INT64_MIN};
    switch (below(4)) {
        case 0: return edges[below((int64_t)(sizeof edges / sizeof edges[0]))];
        case 1: return below(100);
        case 2: return below((int64_t)1 << below(63));
        default:   /* a neighbour, wrapping at the int64 limits (no signed overflow) */
            return (int64_t)((uint64_t)edges[below((int64_t)(sizeof edges / sizeof edges[0]))] +
                             (uint64_t)(below(5) - 2));
    }
}

static void *fuzz_ptr(void)
{
    static const uintptr_t choices[] = {0, FAKE, FAKE + 1, FAKE + 4, FAKE + 8, FAKE + 16,
                                        FAKE + 4096, (uintptr_t)1 << 40, ((uintptr_t)1 << 47) - 16};
    /* mostly aligned, non-null */
    return below(4) ? P(FAKE + 4096 * (uintptr_t)below(16))
                    : P(choices[below((int64_t)(sizeof choices / sizeof choices[0]))]);
}

static int fuzz_dtype(void) { return below(8) ? (int)below(2) : (int)below(5) - 1; }

static long launched_calls, rc_count[5];

static void record(int rc, long launches_before)
{
    if (rc < 0 || rc > 4) {
        fprintf(stderr, "return code %d out of range\n", rc);
        ++failures;
        return;
    }
    ++rc_count[rc];
    if (rc == PSQ_OK) {
        if (stub_launches == launches_before) {
            fprintf(stderr, "a successful call launched nothing\n");
            ++failures;
        }
        ++launched_calls;
    }
}

/* the query/call consistency of one entry point: q = the query for these
 * sizes; the call is made with a good workspace of q bytes, then q-1 */
#define WS_CONSISTENCY(q, CALL, a)                                                      \
    do {                                                                                \
        long ws_l0 = stub_launches;                                                     \
        int ws_rc;                                                                      \
        (a).ws = P(FAKE);                                                               \
        (a).wsb = (q) ? (q) : ((size_t)1 << 40);                                        \
        ws_rc = CALL(a);                                                                \
        record(ws_rc, ws_l0);                                                           \
        if ((q) == 0 && ws_rc != PSQ_ERR_ARG && ws_rc != PSQ_ERR_OVERFLOW) {            \
            fprintf(stderr, "line %d: query 0 but call returned %d\n", __LINE__, ws_rc); \
            ++failures;                                                                 \
        }                                                                               \
        if ((q) > 0 && ws_rc == PSQ_OK) {                                               \
            (a).wsb = (q) - 1;                                                          \
            ws_l0 = stub_launches;                                                      \
            ws_rc = CALL(a);                                                            \
            ++rc_count[3];                                                              \
            if (ws_rc != PSQ_ERR_WORKSPACE || stub_launches != ws_l0) {                 \
                fprintf(stderr, "line %d: one byte short returned %d\n", __LINE__, ws_rc); \
                ++failures;                                                             \
            }                                                                           \
            (a).wsb = (q);                                                              \
            (a).ws = P(FAKE + 8);                                                       \
            ws_rc = CALL(a);                                                            \
            if (ws_rc != PSQ_ERR_WORKSPACE || stub_launches != ws_l0) {                 \
                fprintf(stderr, "line %d: misaligned returned %d\n", __LINE__, ws_rc);  \
                ++failures;                                                             \
            }                                                                           \
        }                                                                               \
    } while (0)

static void fuzz_copies(psq_copy *c, int *n)
{
    int i;
    *n = below(6) ? (int)below(4) : (int)below(11) - 1;
    for (i = 0; i < 10; ++i) {
        uintptr_t src = (uintptr_t)fuzz_ptr();
        uintptr_t dst = below(5) ? src + (uintptr_t)edge_size() : (uintptr_t)fuzz_ptr();
        int64_t rows = below(3) ? below(5) : edge_size();
        int64_t row = below(3) ? 16 * below(64) : edge_size();
        int64_t sst = below(2) ? row : edge_size();
        int64_t dst_st = below(3) ? 0 : edge_size();
        c[i] = copy_of(src, dst, rows, row, sst, dst_st);
    }
}

static void fuzz_one(void)
{
    const int which = (int)below(7);
    long l0 = stub_launches;
    int rc;
    if (which == 0) {
        DocA a = doc_defaults();
        a.doc = below(8) ? P(FAKE) : fuzz_ptr();
        a.dt = fuzz_dtype();
        a.B = below(3) ? below(1 << 12) : edge_size();
        a.S = below(3) ? below(1 << 16) : edge_size();
        a.mask = below(2) ? NULL : fuzz_ptr();
        {
            size_t q = psq_params_from_doc_ids_workspace(a.B, a.S);
            WS_CONSISTENCY(q, doc_call, a);
        }
        l0 = stub_launches;
        rc = noalloc_call(a);
        record(rc, l0);
    } else if (which == 1 || which == 2) {
        psq_thd_layout lay;
        psq_copy c[10];
        int n;
        ThdA a;
        if (which == 1)
            lay = layout(below(10) ? PSQ_LAYOUT_SEQ_LENS : (int)below(4), fuzz_ptr(),
                         below(2) ? NULL : fuzz_ptr(), fuzz_dtype(),
                         below(3) ? below(300) : edge_size(), below(4) ? -1000 : edge_size(),
                         NULL, PSQ_I32);
        else
            lay = doc_layout(below(8) ? P(FAKE) : fuzz_ptr(), fuzz_dtype());
        a = thd_defaults(below(50) ? &lay : NULL);
        a.B = below(3) ? below(1 << 14) : edge_size();
        a.S = below(3) ? below(1 << 16) : edge_size();
        a.cp = below(2) ? NULL : fuzz_ptr();
        a.mask = below(2) ? NULL : fuzz_ptr();
        fuzz_copies(c, &n);
        a.copies = below(20) ? c : NULL;
        a.n_copies = n;
        {
            size_t q = a.lay ? psq_process_thd_workspace(a.lay, a.B, a.S) : 0;
            WS_CONSISTENCY(q, thd_call, a);
        }
    } else if (which == 3) {
        psq_thd_layout lay = layout(below(10) ? PSQ_LAYOUT_SEQ_LENS : (int)below(4), fuzz_ptr(),
                                    below(2) ? NULL : fuzz_ptr(), fuzz_dtype(),
                                    below(3) ? below(300) : edge_size(),
                                    below(4) ? -1000 : edge_size(), NULL, PSQ_I32);
        SplitA a = split_defaults(&lay);
        a.B = below(3) ? 1 + below(1 << 12) : edge_size();
        a.S = below(3) ? below(1 << 16) : edge_size();
        a.G = below(3) ? 1 + below(64) : edge_size();
        if (below(2) && a.G > 0 && a.G < ((int64_t)1 << 40)) a.B = a.G * (1 + below(8));
        a.cp = below(2) ? NULL : fuzz_ptr();
        {
            size_t q = psq_split_thd_workspace(&lay, a.B, a.S, a.G);
            WS_CONSISTENCY(q, split_call, a);
        }
    } else if (which == 4) {
        PadA a = pad_defaults();
        a.dt = fuzz_dtype();
        a.T = below(3) ? below(1 << 20) : edge_size();
        a.pad = edge_size();
        a.nc = below(2) ? NULL : fuzz_ptr();
        {
            size_t q = psq_padding_mask_from_token_ids_workspace(a.T);
            WS_CONSISTENCY(q, pad_call, a);
        }
    } else if (which == 5) {
        PackA a = pack_defaults();
        a.src_len = edge_size();
        a.N = below(3) ? below(1 << 16) : edge_size();
        a.P_ = below(3) ? below(1 << 12) : edge_size();
        a.q = (int32_t)(below(3) ? 1 + below(128) : edge_size());
        a.C = (int32_t)(below(3) ? 1 + below(1 << 16) : edge_size());
        a.fold = (int)below(2);
        a.order = below(2) ? NULL : fuzz_ptr();
        {
            size_t q = psq_pack_rows_workspace(a.N, a.P_, a.C);
            WS_CONSISTENCY(q, pack_call, a);
        }
    } else {
        RectA a = rect_defaults();
        a.W = below(3) ? below(1 << 14) : edge_size();
        a.N = below(3) ? below(1 << 12) : edge_size();
        a.P_ = below(3) ? below(1 << 10) : edge_size();
        a.q = (int32_t)(below(3) ? 1 + below(128) : edge_size());
        a.C = (int32_t)(below(3) ? 1 + below(1 << 16) : edge_size());
        a.order = below(2) ? NULL : fuzz_ptr();
        {
            size_t q = psq_pack_rows_workspace(a.N, a.P_, a.C);
            WS_CONSISTENCY(q, rect_call, a);
        }
    }
    (void)psq_status_string((int)below(600) - 50, (int)below(2));
}

int main(int argc, char **argv)
{
    long iters = argc > 1 ? atol(argv[1]) : 10000, i;
    rng_state = 0x9E3779B97F4A7C15ull ^ (uint64_t)(argc > 2 ? atol(argv[2]) : 1);
    host_test_cases();
    for (i = 0; i < iters; ++i) fuzz_one();
    if (failures) {
        fprintf(stderr, "%ld of %ld checks failed\n", failures, checks);
        return 1;
    }
    printf("ok %ld checks %ld launched %ld ok %ld arg %ld overflow %ld workspace %ld hip %ld\n",
           iters, checks, launched_calls, rc_count[0], rc_count[1], rc_count[2], rc_count[3],
           rc_count[4]);
    return 0;
}
