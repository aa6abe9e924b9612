/*
 * uniprefill_prof.h - instrumentation entry point of libuniprefill.
 *
 * Not part of the selection path's interface (include/uniprefill.h): a
 * benchmark uses it to time the score GEMM on its own while the rest of
 * up_select_blocks runs as usual.
 */
#ifndef UNIPREFILL_PROF_H
#define UNIPREFILL_PROF_H

#include "uniprefill.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * up_select_blocks_profiled - up_select_blocks (same arguments, same work and
 * results, same validation), and additionally records the hipEvent_t handles
 * score_begin and score_end on `stream` immediately before and immediately
 * after the score kernel (UniPrefill Sec. 3.5 Eq. 13, the partial GEMM with the
 * first pass of the online softmax), so hipEventElapsedTime(score_begin,
 * score_end) brackets that one kernel.  Either event may be NULL (not
 * recorded).  With UP_SCORES_IN there is no score kernel and neither event is
 * recorded.  The events are the caller's; a failed hipEventRecord returns
 * UP_ERR_HIP.
 */
up_status up_select_blocks_profiled(const up_select_params* prm,
                                    const void* q, int64_t q_row_stride,
                                    const void* k, int64_t k_row_stride,
                                    const int32_t* cu_seqlens, int32_t num_reqs, int64_t max_tokens,
                                    const float* scores_in,
                                    float* block_scores, int32_t* block_offsets,
                                    uint8_t* keep_block, uint8_t* keep_mask, int32_t* kept_per_req,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    void* score_begin, void* score_end);

#ifdef __cplusplus
}
#endif

#endif /* UNIPREFILL_PROF_H */
