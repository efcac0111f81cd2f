/* ep_oracle.h -- the oracle's own interface.
 *
 * TEST INFRASTRUCTURE ONLY. This header belongs to the CPU oracle under oracle/
 * and is included by nothing outside oracle/. The GPU library has its own
 * header (include/ep.h); the two share no declarations, constants or code.
 *
 * All arrays are host memory, row-major, owned by the caller.
 * Status bits returned by the functions below (values chosen equal to the
 * library's sticky status bits so that tests can compare them directly):
 *   1 = an expert id outside [-1, E), 2 = a repeated expert within one token,
 *   4 = some rank receives more rows than cap_rows.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_ST_BAD_EXPERT 1u
#define ORACLE_ST_DUP_EXPERT 2u
#define ORACLE_ST_CAPACITY 4u

uint32_t oracle_layout(int T, int k, int E, int R, long long cap_rows,
                       const int32_t *topk_idx,
                       int32_t *cnt_se, int32_t *cnt_sd, int32_t *recv_cnt,
                       int32_t *expert_off, int32_t *rank_rows,
                       int32_t *src_expert_off, int32_t *rank_in_expert,
                       uint8_t *is_token_in_rank);

void oracle_positions(int T, int k, int E, int R, long long cap_rows,
                      const int32_t *topk_idx, const int32_t *rank_in_expert,
                      const int32_t *expert_off, int32_t *pos, int32_t *src_idx);

void oracle_dispatch(int T, int k, int H, int use_fp8, const uint16_t *x,
                     const float *topk_w, const int32_t *pos,
                     const int32_t *tokens, int ntokens,
                     void *recv_x, float *recv_scales, float *recv_w);

void oracle_quantize_token(int H, const uint16_t *x_row, uint8_t *q, float *scales);

uint32_t oracle_layout_dedup(int T, int k, int E, int R, long long cap_rows,
                             const int32_t *topk_idx, int32_t *rank_in_rank, int32_t *token_rows);

uint32_t oracle_ll_positions(int T, int k, int E, int R, const int32_t *topk_idx,
                             int32_t *pos, int32_t *src_idx, int32_t *recv_count);

void oracle_positions_dedup(int T, int k, int E, int R, long long cap_rows,
                            const int32_t *topk_idx, const int32_t *rank_in_rank,
                            int32_t *pos, int32_t *src_idx);

void oracle_dispatch_dedup(int T, int k, int H, int E, int R, int use_fp8, const uint16_t *x,
                           const int32_t *topk_idx, const float *topk_w, const int32_t *pos,
                           const int32_t *tokens, int ntokens, void *recv_x, float *recv_scales,
                           int32_t *recv_topk_idx, float *recv_topk_w);

void oracle_combine(int T, int k, int H, const uint16_t *rows, const int32_t *pos,
                    const float *w, const int32_t *tokens, int ntokens,
                    uint16_t *y, float *acc);

void oracle_prereduce(int R, long long cap_rows, int k, int H, long long row_lo, long long row_hi,
                      const uint16_t *expert_out, const int32_t *recv_topk_idx,
                      const float *recv_topk_w, const int32_t *token_rows,
                      uint16_t *reduced, float *sums);

void oracle_combine_backward(int T, int k, int H, const uint16_t *grad_y,
                             const int32_t *pos, uint16_t *grad_rows);

void oracle_e4m3_encode(const float *in, uint8_t *out, long long n);
void oracle_e4m3_decode(const uint8_t *in, float *out, long long n);
void oracle_bf16_round(const float *in, uint16_t *out, long long n);

#ifdef __cplusplus
}
#endif
#endif
