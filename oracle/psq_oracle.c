/*
 * psq_oracle.c -- plain, slow, single-threaded CPU oracle for packed-sequence
 * (THD) varlen-attention metadata.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library: it is written directly from the three pages it cites.
 *
 * Every function is a literal transcription of a definition, with no
 * blocking, fusion or reordering: one loop per step, in the order the pages
 * give the steps.  Integer results are exact, so the GPU path must match
 * them bit for bit.
 *
 * Pages cited:
 *   [P1] NeMo AutoModel API reference, "nemo_automodel.components.datasets.
 *        packed_seq" (module text; PackedSeqParams; packed_seq_params_from_doc_ids).
 *   [P2] NeMo AutoModel 0.5 API reference, "nemo_automodel.components.
 *        distributed.thd_utils" (_thd_padding_mask; process_input_for_thd,
 *        its Example and Returns).
 *        Also thd_padding_mask_from_token_ids and split_batch_into_thd_chunks
 *        (the latter is assembled from orc_thd_tables in oracle/__init__.py).
 *   [P3] "Who packs the sequences: the loader, or the trainer?" (sections
 *        "What the data looks like at each hop": Trainer packs / Loader packs).
 *
 * Status bits (data-dependent errors).  A function returns the OR of every
 * condition that holds; outputs are unspecified when the result is non-zero.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BAD_LENGTH      1u   /* negative length, or real > padded          */
#define ORC_TABLE_MISMATCH  2u   /* sentinel positions differ between tables   */
#define ORC_ROW_OVERFLOW    4u   /* padded lengths of a row exceed the row     */
#define ORC_EMPTY_ROW       8u   /* a row holds no sequence                    */
#define ORC_PACK_OVERFLOW  16u   /* padded sources exceed the pack capacity    */
#define ORC_EMPTY_PACK     32u   /* a pack has no member                       */
#define ORC_BAD_INDEX      64u   /* member / pack / source range out of bounds */
#define ORC_PAD_IS_CONTENT 256u   /* the pad id also occurs before the pad tail */

/* malloc that never returns NULL: an oracle that cannot hold its scratch */
/* arrays stops the test run instead of returning a wrong answer.        */
static void *orc_alloc(size_t bytes)
{
    void *p = malloc(bytes > 0 ? bytes : 1);
    if (p == NULL) {
        fprintf(stderr, "psq oracle: out of memory (%zu bytes)\n", bytes);
        abort();
    }
    return p;
}

/* ------------------------------------------------------------------------ */
/* [P1] packed_seq_params_from_doc_ids.                                      */
/*                                                                          */
/* Segments are the maximal runs of one document index inside a row, and a   */
/* new segment always starts at the beginning of a row (module text: the     */
/* flattened batch must not merge a row-filling document with the next row's */
/* first document).  Padding runs (index 0) are segments too.  cu_seqlens    */
/* holds the start of every segment over the flattened B*S axis followed by  */
/* B*S (PackedSeqParams.cu_seqlens), and max_seqlen is the longest segment   */
/* (PackedSeqParams.max_seqlen).  The padding mask marks index 0.            */
/*                                                                          */
/* doc:  B*S document indices, row-major, widened to int64 by the caller.    */
/* cu:   room for B*S+1 entries.  mask: B*S bytes or NULL.                   */
/* Returns the number of segments; cu[0..nseg] is valid.                     */
/* ------------------------------------------------------------------------ */
int64_t orc_doc_segments(const int64_t *doc, int64_t B, int64_t S,
                         int32_t *cu, int32_t *max_seqlen, uint8_t *mask)
{
    int64_t T = B * S;
    int64_t nseg = 0;
    int64_t t, k;
    int32_t best = 0;

    /* Step 1: list the segment starts. */
    for (t = 0; t < T; t++) {
        int starts_row = (t % S) == 0;
        int new_doc = (t > 0) && (doc[t] != doc[t - 1]);
        if (starts_row || new_doc) {
            cu[nseg] = (int32_t)t;
            nseg++;
        }
    }
    /* Step 2: close the last segment at the end of the flattened axis. */
    cu[nseg] = (int32_t)T;

    /* Step 3: the longest segment, padding runs included. */
    for (k = 0; k < nseg; k++) {
        int32_t len = cu[k + 1] - cu[k];
        if (len > best)
            best = len;
    }
    *max_seqlen = best;

    /* Step 4: padding is document index 0. */
    if (mask != NULL) {
        for (t = 0; t < T; t++)
            mask[t] = (uint8_t)(doc[t] == 0);
    }
    return nseg;
}

/* ------------------------------------------------------------------------ */
/* [P2] process_input_for_thd on per-row sequence tables, with               */
/* _thd_padding_mask.                                                        */
/*                                                                          */
/* L[B][P]  : real lengths (seq_lens), v marks an unused slot.               */
/* Lp[B][P] : slot counts (seq_lens_padded), same sentinel, or NULL.         */
/*                                                                          */
/* Readings of the page taken here (the page leaves these steps open):       */
/*  - a row's trailing pad (S minus the sum of its padded lengths) is folded */
/*    into that row's last sequence, so the physical boundaries of row r end */
/*    at (r+1)*S and every sequence sits where its tokens are;               */
/*  - the absorption gate fires when every interior boundary of the real     */
/*    array equals the physical one and the real array ends before T; it     */
/*    then sets the last real boundary to T;                                 */
/*  - max_seqlen is the largest step of cu_seqlens after absorption (the     */
/*    Returns formula);                                                      */
/*  - the padding mask is taken from the physical layout before absorption:  */
/*    sequence i owns [cp[i], cp[i]+real_i) as tokens, everything else pads. */
/*  - without Lp, each sequence reserves exactly its real length.            */
/*                                                                          */
/* The page prints no case where a row's padded lengths fall short of S, or  */
/* where absorption fires: those two readings are parity unpinned by any     */
/* printed value.  The tests pin them by invariants, hand cases and an       */
/* independent slot-grid formulation of the same readings.                   */
/*                                                                          */
/* cu, cp: room for B*P+1 entries.  mask: B*S bytes.                         */
/* Returns the status bits; *nseq, *max_seqlen, *pad_between on success.     */
/* ------------------------------------------------------------------------ */
uint32_t orc_thd_tables(const int64_t *L, const int64_t *Lp,
                        int64_t B, int64_t P, int64_t S, int64_t v,
                        int32_t *cu, int32_t *cp, int64_t *nseq,
                        int32_t *max_seqlen, int32_t *pad_between,
                        uint8_t *mask)
{
    uint32_t status = 0;
    int64_t T = B * S;
    int64_t r, j, i, t, n;
    int64_t *real, *phys;

    *nseq = 0;
    *max_seqlen = 0;
    *pad_between = 0;

    /* Validation: sentinels must line up, lengths must be sane, every row */
    /* must hold a sequence and its padded lengths must fit the row.       */
    for (r = 0; r < B; r++) {
        int64_t count = 0;
        int64_t padded_sum = 0;          /* of clamp(Lp, 0, S+1): no overflow */
        for (j = 0; j < P; j++) {
            int64_t l = L[r * P + j];
            int64_t lp = (Lp != NULL) ? Lp[r * P + j] : l;
            int valid = (l != v);
            if (Lp != NULL && ((lp != v) != valid))
                status |= ORC_TABLE_MISMATCH;
            if (!valid)
                continue;
            count++;
            if (l < 0 || lp < l)
                status |= ORC_BAD_LENGTH;
            if (lp > 0)
                padded_sum += (lp > S) ? S + 1 : lp;
        }
        if (count == 0)
            status |= ORC_EMPTY_ROW;
        if (padded_sum > S)
            status |= ORC_ROW_OVERFLOW;
    }
    if (status != 0)
        return status;

    /* Step 1: keep the valid entries in row-major order (sentinel filter). */
    real = (int64_t *)orc_alloc(sizeof(int64_t) * (size_t)(B * P + 1));
    phys = (int64_t *)orc_alloc(sizeof(int64_t) * (size_t)(B * P + 1));
    n = 0;
    for (r = 0; r < B; r++) {
        int64_t row_used = 0;
        int64_t last = -1;
        for (j = 0; j < P; j++) {
            int64_t l = L[r * P + j];
            if (l == v)
                continue;
            real[n] = l;
            phys[n] = (Lp != NULL) ? Lp[r * P + j] : l;
            row_used += phys[n];
            last = n;
            n++;
        }
        /* Step 2: fold the row's trailing pad into its last sequence. */
        phys[last] += S - row_used;
    }

    /* Step 3: cumulative real and physical boundaries. */
    cu[0] = 0;
    cp[0] = 0;
    for (i = 0; i < n; i++) {
        cu[i + 1] = cu[i] + (int32_t)real[i];
        cp[i + 1] = cp[i] + (int32_t)phys[i];
    }

    /* Step 4: padding mask from the layout (_thd_padding_mask). */
    for (t = 0; t < T; t++)
        mask[t] = 1;
    for (i = 0; i < n; i++) {
        for (t = cp[i]; t < cp[i] + real[i]; t++)
            mask[t] = 0;
    }

    /* Step 5: trailing-pad absorption (single context-parallel rank). */
    {
        int interior_agree = 1;
        for (i = 1; i < n; i++) {
            if (cu[i] != cp[i])
                interior_agree = 0;
        }
        if (interior_agree && cu[n] < T)
            cu[n] = (int32_t)T;
    }

    /* Step 6: do the two arrays differ, and the widest real step. */
    for (i = 0; i <= n; i++) {
        if (cu[i] != cp[i])
            *pad_between = 1;
    }
    for (i = 0; i < n; i++) {
        int32_t step = cu[i + 1] - cu[i];
        if (step > *max_seqlen)
            *max_seqlen = step;
    }
    *nseq = n;

    free(real);
    free(phys);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* [P2] process_input_for_thd, the collapse of a [B,S,...] tensor to         */
/* [B*S,...]: the bytes do not change, only the shape.  Rows may sit at a    */
/* stride in the source; the destination is dense.                          */
/* ------------------------------------------------------------------------ */
void orc_copy_rows(const uint8_t *src, uint8_t *dst, int64_t rows,
                   int64_t row_bytes, int64_t src_row_stride_bytes)
{
    int64_t r, b;
    for (r = 0; r < rows; r++) {
        for (b = 0; b < row_bytes; b++)
            dst[r * row_bytes + b] = src[r * src_row_stride_bytes + b];
    }
}

/* ------------------------------------------------------------------------ */
/* [P3] the squeeze into fixed-capacity packs.                               */
/*                                                                          */
/* Each source is padded to a multiple of q, the padded sources of a pack    */
/* are laid end to end (Trainer packs: [0,5,15] real, [0,8,20] padded), the  */
/* rest of the row up to capacity is pad, token_mask is 1 exactly on real    */
/* tokens (Loader packs), and with fold the last padded boundary becomes    */
/* the capacity (Loader packs: [0,8,36]).                                    */
/*                                                                          */
/* Members of pack p are entries pack_start[p] .. pack_start[p+1]-1 of       */
/* order (or those source indices themselves when order is NULL).  Source i  */
/* is src[src_off[i] .. src_off[i]+real_len[i]).  Per-pack boundary arrays   */
/* are stored one after another: pack p's k+1 entries start at               */
/* pack_start[p] + p.                                                        */
/* ------------------------------------------------------------------------ */
/* row_width >= 0: the sources are the rows of a rectangle that wide, and a */
/* length beyond it is a BAD_LENGTH (the trainer path, orc_pack_rect).       */
static uint32_t pack_impl(const int64_t *src, int64_t src_len, const int64_t *src_off,
                          const int32_t *real_len, int64_t N, int32_t q,
                          const int32_t *order, const int64_t *pack_start, int64_t P,
                          int32_t C, int fold, int64_t pad_token,
                          int64_t *packed, uint8_t *token_mask,
                          int32_t *cu, int32_t *cp, int64_t row_width)
{
    uint32_t status = 0;
    int64_t p, j, s;

    /* Validation. */
    for (p = 0; p < P; p++) {
        int64_t a = pack_start[p];
        int64_t b = pack_start[p + 1];
        int64_t used = 0;
        if (a < 0 || b > N || b < a) {
            status |= ORC_BAD_INDEX;
            continue;
        }
        if (b == a)
            status |= ORC_EMPTY_PACK;
        for (j = a; j < b; j++) {
            int64_t i = (order != NULL) ? (int64_t)order[j] : j;
            int64_t real;
            if (i < 0 || i >= N) {
                status |= ORC_BAD_INDEX;
                continue;
            }
            real = real_len[i];
            if (real < 0 || (row_width >= 0 && real > row_width)) {
                status |= ORC_BAD_LENGTH;
                continue;
            }
            if (src_off[i] < 0 || src_off[i] > src_len - real)
                status |= ORC_BAD_INDEX;
            used += (real + q - 1) / q * q;
        }
        if (used > C)
            status |= ORC_PACK_OVERFLOW;
    }
    if (status != 0)
        return status;

    for (p = 0; p < P; p++) {
        int64_t a = pack_start[p];
        int64_t b = pack_start[p + 1];
        int64_t k = b - a;
        int32_t *pcu = cu + a + p;
        int32_t *pcp = cp + a + p;
        int64_t *row = packed + p * (int64_t)C;
        uint8_t *mrow = token_mask + p * (int64_t)C;
        int64_t off = 0;

        pcu[0] = 0;
        pcp[0] = 0;
        for (j = 0; j < k; j++) {
            int64_t i = (order != NULL) ? (int64_t)order[a + j] : a + j;
            int64_t real = real_len[i];
            int64_t padded = (real + q - 1) / q * q;
            /* the source's tokens */
            for (s = 0; s < real; s++) {
                row[off + s] = src[src_off[i] + s];
                mrow[off + s] = 1;
            }
            /* the source's own pad */
            for (s = real; s < padded; s++) {
                row[off + s] = pad_token;
                mrow[off + s] = 0;
            }
            off += padded;
            pcu[j + 1] = pcu[j] + (int32_t)real;
            pcp[j + 1] = (int32_t)off;
        }
        /* tail pad up to capacity */
        for (s = off; s < C; s++) {
            row[s] = pad_token;
            mrow[s] = 0;
        }
        /* fold: the last padded boundary is the capacity */
        if (fold)
            pcp[k] = C;
    }
    return 0;
}

uint32_t orc_pack(const int64_t *src, int64_t src_len, const int64_t *src_off,
                  const int32_t *real_len, int64_t N, int32_t q,
                  const int32_t *order, const int64_t *pack_start, int64_t P,
                  int32_t C, int fold, int64_t pad_token,
                  int64_t *packed, uint8_t *token_mask,
                  int32_t *cu, int32_t *cp)
{
    return pack_impl(src, src_len, src_off, real_len, N, q, order, pack_start, P, C,
                     fold, pad_token, packed, token_mask, cu, cp, -1);
}

/* ------------------------------------------------------------------------ */
/* [P3] Trainer packs: the squeeze straight from the padded rectangle the    */
/* worker receives (input_ids [N, W] with input_lengths), bins chosen on the  */
/* host.  Row i holds source i in its first real_len[i] slots, so the source */
/* offsets are i*W, and a member whose length is negative or beyond the row  */
/* is a BAD_LENGTH.  Everything else is orc_pack (the trainer path runs it   */
/* without the fold).                                                        */
/* ------------------------------------------------------------------------ */
uint32_t orc_pack_rect(const int64_t *rows, int64_t W, const int32_t *real_len,
                       int64_t N, int32_t q, const int32_t *order,
                       const int64_t *pack_start, int64_t P, int32_t C, int fold,
                       int64_t pad_token, int64_t *packed, uint8_t *token_mask,
                       int32_t *cu, int32_t *cp)
{
    uint32_t status;
    int64_t i;
    int64_t *off;

    off = (int64_t *)orc_alloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    for (i = 0; i < N; i++)
        off[i] = i * W;
    status = pack_impl(rows, N * W, off, real_len, N, q, order, pack_start, P, C,
                       fold, pad_token, packed, token_mask, cu, cp, W);
    free(off);
    return status;
}

/* ------------------------------------------------------------------------ */
/* [P2] thd_padding_mask_from_token_ids: the metadata-free mask.             */
/*                                                                          */
/* A slot is padding when its id equals the pad id.  That comparison gives  */
/* the right mask only if the pad slots are one run that ends the stream,   */
/* so the stream is checked for exactly that: from the first pad slot on,    */
/* every slot must be pad.  Otherwise the pad id is also content (the        */
/* page's pad == end-of-text case) and the call fails.                       */
/*                                                                          */
/* ids: T token ids.  mask: T bytes.  *num_content: index of the first pad   */
/* slot (T when there is none), i.e. the length of the content prefix.       */
/* ------------------------------------------------------------------------ */
uint32_t orc_pad_mask_from_ids(const int64_t *ids, int64_t T, int64_t pad,
                               uint8_t *mask, int64_t *num_content)
{
    uint32_t status = 0;
    int64_t t, first_pad = T;

    /* Step 1: the value comparison. */
    for (t = 0; t < T; t++)
        mask[t] = (uint8_t)(ids[t] == pad);

    /* Step 2: find where the tail would begin ... */
    for (t = 0; t < T; t++) {
        if (mask[t]) {
            first_pad = t;
            break;
        }
    }
    /* ... and reject a non-pad id after it. */
    for (t = first_pad; t < T; t++) {
        if (!mask[t])
            status |= ORC_PAD_IS_CONTENT;
    }
    *num_content = first_pad;
    return status;
}
