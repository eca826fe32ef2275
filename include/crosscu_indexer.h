/*
 * crosscu indexer: paged indexer score and top-k selection, the step that
 * produces the index sets of index-sparse decode attention (GLM-5.2 decode
 * article: the decode layer runs "Paged Indexer Score" before TopK and sparse
 * MLA, Summary; the indexer rank computes the scores and the Top-2048 and
 * publishes the indices to the attention ranks, related-work section on
 * TileRT).  The pages name these steps, not the score's formula; this library
 * computes, for decode token t of request b and cached token j < L_b:
 *
 *   score(t, j) = sum_i q[b, t, i] * k[j, i]      (one indexer head, dim 128)
 *
 * in fp32: each product of two bf16 values is exact in fp32 and is added to
 * the running sum for i = 0 .. 127 in index order, one rounding per addition.
 * indices[b, t, :] are the topk positions j of largest score, ties to the
 * lower position, listed in increasing order.
 *
 * Conventions (return codes, ownership, host vs device, streams) as in
 * crosscu.h.
 */
#ifndef CROSSCU_INDEXER_H
#define CROSSCU_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch;              /* B requests, 1 .. 64                          */
  int32_t q_tokens;           /* Tq decode tokens per request, 1 .. 16        */
  int32_t dim;                /* indexer head dimension; 128 is implemented   */
  int32_t page_size;          /* tokens per page, a power of two              */
  int32_t max_pages_per_seq;  /* columns of block_table                       */
  int32_t num_pages;          /* pages in k_cache                             */
  int32_t topk;               /* positions kept per decode token              */
} cc_indexer_problem;

/* Bytes of the fp32 score scratch cc_indexer_topk needs for these lengths:
 * B * Tq * max_b(L_b) * 4.  seqlens: host int32[B].  Returns CC_OK or
 * CC_ERR_INVALID. */
int cc_indexer_scratch_size(const cc_indexer_problem* p, const int32_t* seqlens, size_t* bytes);

/* Scores every cached token of each request against that request's decode
 * tokens, then writes each decode token's top-k positions.
 *   seqlens      host int32[B]: 1 <= L_b <= 16384 and topk <= L_b
 *   q            device bf16 [B, Tq, dim]: indexer queries
 *   k_cache      device bf16 [num_pages, page_size, dim]: indexer keys
 *   block_table  device int32 [B, max_pages_per_seq]: token j of request b is
 *                row j % page_size of page block_table[b, j / page_size];
 *                ceil(L_b / page_size) <= max_pages_per_seq (checked)
 *   scratch      device, >= cc_indexer_scratch_size bytes: fp32 scores
 *                [B * Tq, max L_b], overwritten
 *   indices      device int32 [B, Tq, topk]: written, increasing positions
 *                (the index layout cc_decode takes in CC_MODE_MLA_SPARSE)
 *   err          device int32 or NULL: bit value 2 is OR-ed in when a used
 *                block_table entry lies outside [0, num_pages); such a row
 *                is read from the nearest valid page
 * Two kernels on `stream`; nothing is allocated.  Returns CC_OK,
 * CC_ERR_INVALID, CC_ERR_UNSUPPORTED (dim != 128, Tq > 16, B > 64,
 * L_b > 16384), CC_ERR_BUFFER (scratch too small) or CC_ERR_HIP. */
int cc_indexer_topk(const cc_indexer_problem* p, const int32_t* seqlens, const void* q, const void* k_cache,
                    const int32_t* block_table, void* scratch, size_t scratch_bytes, int32_t* indices, int32_t* err,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CROSSCU_INDEXER_H */
