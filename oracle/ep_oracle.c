/* ep_oracle.c -- CPU oracle for the MoE dispatch / combine hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this code. The GPU library never includes, links or
 * calls it, and it shares no code, header, table or helper with the GPU path.
 *
 * Plain, slow, single-threaded C99 written to be checked by eye. Every
 * function below computes the plain definition of its step directly:
 *   - layout: per-expert / per-rank counts and a stable counting sort of the
 *     (token, slot) entries by expert, done with one sequential counter per
 *     expert (no scan, no tiling);
 *   - dispatch: a copy of each token's row to its receive rows, optionally
 *     quantized to OCP FP8 e4m3 with one fp32 scale per 128 channels;
 *   - combine: a weighted sum of the token's received rows in fp32, one fused
 *     multiply-add per slot in slot order, rounded once to bf16.
 *
 * Sources. The operations and their inputs/outputs are the ones the DeepEP
 * usage guide (zhouruolin.cn, "DeepEP：MoE 专家并行 EP 通信 kernel 编译与使用指南",
 * section 5 "使用方法") gives for dispatch(x, topk_idx, topk_weights,
 * num_experts, ...) -> (recv_x, _, recv_topk_weights, handle), for
 * combine(expert_output, handle) -> combined_x, and for reusing the handle in
 * combine_backward / dispatch_backward. "FP8 dispatch + BF16 combine" is the
 * precision pairing given in the blog.hotdry.top DeepEP notes (section 5,
 * precision choice) and in the czhn.yksolo.com launch report (normal-kernel
 * setup). Everything the pages leave open (receive layout, slot order, FP8
 * scale formula, rounding, combine arithmetic) follows the readings listed in
 * the design doc; each is restated at the function that uses it.
 *
 * Parity pins: each function is pinned by tests under tests/ (test_oracle_*).
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

static float f32_from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bfloat16 -> float: a bf16 value is the top 16 bits of the fp32 pattern. */
static float bf16_to_float(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Magnitude (as a double) of the fp32 pattern u, with +-Inf standing for the
 * first power of two past the largest finite value (2^128), which is how IEEE
 * round-to-nearest decides overflow. */
static double magnitude_for_rounding(uint32_t u) {
    if ((u & 0x7fffffffu) == 0x7f800000u) return ldexp(1.0, 128);
    return fabs((double)f32_from_bits(u));
}

/* float -> bfloat16, round to nearest, ties to even (IEEE 754 default mode).
 * Written as the definition: of the two bf16 neighbours of f (truncation
 * toward zero, and the next value away from zero) take the nearer one; on an
 * exact tie take the one whose last mantissa bit is 0. */
static uint16_t bf16_from_float(float f) {
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u); /* keep it a quiet NaN */
    uint32_t lo = u & 0xffff0000u;
    if (lo == u) return (uint16_t)(u >> 16);
    uint32_t hi = lo + 0x00010000u; /* next bf16 away from zero (may be Inf) */
    double a = fabs((double)f);
    double d_lo = a - magnitude_for_rounding(lo);
    double d_hi = magnitude_for_rounding(hi) - a;
    if (d_lo < d_hi) return (uint16_t)(lo >> 16);
    if (d_hi < d_lo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest finite
 * magnitude 1.75 * 2^8 = 448, subnormals m * 2^-9 for exponent field 0. */
static float e4m3_to_float(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return s ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* float -> e4m3, round to nearest with ties to even, saturating to +-448
 * (satfinite), sign kept (so -0.0 and negative values that round to zero give
 * 0x80). The product inputs are finite; NaN maps to the NaN code.
 * The magnitude a is located in its binade, its scaled mantissa is rounded
 * with nearbyint() in the default round-to-nearest-even mode, and a carry out
 * of the mantissa moves to the next binade. All steps are exact in double. */
static uint8_t e4m3_from_float(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7f);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7e);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: spacing 2^-9; a result of 8 is 2^-6, whose code is
         * exponent field 1, mantissa 0 = 0x08, so the integer is the code. */
        double m = nearbyint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int ex;
    double fr = frexp(a, &ex);         /* a = fr * 2^ex, fr in [0.5, 1) */
    int efield = (ex - 1) + 7;          /* a = (1 + f) * 2^(ex-1) */
    double m = nearbyint((2.0 * fr - 1.0) * 8.0);
    if (m == 8.0) {
        m = 0.0;
        efield += 1;
    }
    int code = (efield << 3) | (int)m;
    if (code > 0x7e) code = 0x7e; /* cannot happen for a < 448; kept as a guard */
    return (uint8_t)(sign | code);
}

void oracle_e4m3_encode(const float *in, uint8_t *out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = e4m3_from_float(in[i]);
}

void oracle_e4m3_decode(const uint8_t *in, float *out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = e4m3_to_float(in[i]);
}

void oracle_bf16_round(const float *in, uint16_t *out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = bf16_from_float(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Layout                                                                      */
/* ------------------------------------------------------------------------- */

/* Is slot j of token t a valid (token, expert) entry?  Reading: -1 marks an
 * empty slot; an id outside [-1, E) is an error (status bit 1) and the slot is
 * dropped; an expert repeated within a token is an error (status bit 2) and
 * every repeat after its first occurrence (in slot order) is dropped. */
static int slot_is_valid(const int32_t *row, int j, int E, uint32_t *status) {
    int32_t e = row[j];
    if (e == -1) return 0;
    if (e < -1 || e >= E) {
        *status |= ORACLE_ST_BAD_EXPERT;
        return 0;
    }
    for (int jj = 0; jj < j; ++jj) {
        if (row[jj] == e) {
            *status |= ORACLE_ST_DUP_EXPERT;
            return 0;
        }
    }
    return 1;
}

/* Dispatch layout.
 * Reading of the simulated expert-parallel group (the pages describe R GPUs
 * exchanging tokens; here R disjoint partitions of one GPU's memory):
 *   source rank of token t:  s(t) = t / (T / R)   (contiguous blocks; T % R == 0)
 *   rank hosting expert e:   d(e) = e / (E / R)   (contiguous blocks; E % R == 0)
 * Outputs:
 *   cnt_se[s][e]          tokens of source rank s routed to expert e
 *   cnt_sd[s][d]          tokens of source rank s with at least one expert on rank d
 *   is_token_in_rank[t][d] 1 if token t has a valid slot whose expert lives on d
 *   recv_cnt[e]           rows expert e receives (sum over s of cnt_se)
 *   expert_off[e]         first row of expert e inside rank d(e)'s region
 *                         (experts of one rank stored in ascending id order)
 *   rank_rows[d]          rows rank d receives
 *   src_expert_off[s][e]  first row, inside rank d(e)'s region, of the rows
 *                         source rank s sends to expert e: expert e's first
 *                         row there plus the rows of e that come from source
 *                         ranks before s. Reading: a sender places its rows in
 *                         the destination rank's receive buffer (the guide's
 *                         dispatch returns each rank's received tokens), so
 *                         the offset it needs is relative to that rank.
 *   rank_in_expert[t][j]  number of tokens t' < t routed to the same expert:
 *                         the stable (by source token index) order of the
 *                         expert's rows; -1 for a slot that is not valid.
 * Returns the status bits (1, 2 from validation, 4 if rank_rows > cap_rows). */
uint32_t oracle_layout(int T, int k, int E, int R, long long cap_rows,
                       const int32_t *topk_idx,
                       int32_t *cnt_se, int32_t *cnt_sd, int32_t *recv_cnt,
                       int32_t *expert_off, int32_t *rank_rows,
                       int32_t *src_expert_off, int32_t *rank_in_expert,
                       uint8_t *is_token_in_rank) {
    uint32_t status = 0;
    int tokens_per_rank = T / R;
    int experts_per_rank = E / R;

    memset(cnt_se, 0, sizeof(int32_t) * (size_t)R * E);
    memset(cnt_sd, 0, sizeof(int32_t) * (size_t)R * R);
    memset(is_token_in_rank, 0, (size_t)T * R);

    /* fill[e] counts the rows of expert e seen so far, in token order */
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t) {
        const int32_t *row = topk_idx + (size_t)t * k;
        int s = t / tokens_per_rank;
        for (int j = 0; j < k; ++j) {
            if (!slot_is_valid(row, j, E, &status)) {
                rank_in_expert[(size_t)t * k + j] = -1;
                continue;
            }
            int e = row[j];
            rank_in_expert[(size_t)t * k + j] = fill[e];
            fill[e] += 1;
            cnt_se[(size_t)s * E + e] += 1;
            is_token_in_rank[(size_t)t * R + e / experts_per_rank] = 1;
        }
        for (int d = 0; d < R; ++d) cnt_sd[(size_t)s * R + d] += is_token_in_rank[(size_t)t * R + d];
    }

    for (int e = 0; e < E; ++e) recv_cnt[e] = fill[e];

    for (int d = 0; d < R; ++d) {
        int32_t off = 0;
        for (int e = d * experts_per_rank; e < (d + 1) * experts_per_rank; ++e) {
            expert_off[e] = off;
            off += recv_cnt[e];
        }
        rank_rows[d] = off;
        if ((long long)off > cap_rows) status |= ORACLE_ST_CAPACITY;
    }

    for (int e = 0; e < E; ++e) {
        int32_t before = 0; /* rows sent to e by source ranks s' < s */
        for (int s = 0; s < R; ++s) {
            src_expert_off[(size_t)s * E + e] = expert_off[e] + before;
            before += cnt_se[(size_t)s * E + e];
        }
    }
    free(fill);
    return status;
}

/* The handle's routing state.
 *   pos[t][j] = d(e) * cap_rows + expert_off[e] + rank_in_expert[t][j]
 * the global receive row of slot (t, j), or -1 if the slot is not valid or its
 * row would fall at or past cap_rows inside rank d(e)'s region (reading: rows
 * beyond the receive capacity are dropped, and the layout reports status 4).
 *   src_idx[pos[t][j]] = t   for every kept slot; other entries untouched. */
void oracle_positions(int T, int k, int E, int R, long long cap_rows,
                      const int32_t *topk_idx, const int32_t *rank_in_expert,
                      const int32_t *expert_off, int32_t *pos, int32_t *src_idx) {
    int experts_per_rank = E / R;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            size_t i = (size_t)t * k + j;
            int32_t e = topk_idx[i];
            int32_t r = rank_in_expert[i];
            if (r < 0 || e < 0 || e >= E) {
                pos[i] = -1;
                continue;
            }
            long long local = (long long)expert_off[e] + r;
            if (local >= cap_rows) {
                pos[i] = -1;
                continue;
            }
            long long p = (long long)(e / experts_per_rank) * cap_rows + local;
            pos[i] = (int32_t)p;
            src_idx[p] = t;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Low-latency receive layout (the low-latency kernels of the blog.hotdry.top
 * DeepEP notes, section 1, and their decode setting: a fixed receive buffer,
 * at most a few hundred tokens per rank, no count exchange before sending).
 * Reading: expert e owns R regions of tpr = T/R rows, region s for source rank
 * s, so a source can place its rows without knowing any other source's
 * counts. A kept slot (t, j) of source s = t / tpr with expert e goes to row
 *   e*R*tpr + s*tpr + (number of earlier tokens of source s routed to e),
 * found here with one counter per (expert, source) while t ascends.
 * pos[t][j] = -1 for a dropped slot; src_idx[row] = t (E*T entries, -1 where
 * unused); recv_count[e][s] = rows used in region (e, s). Returns the status
 * bits of the slots (bad / repeated ids); a region never overflows. */
uint32_t oracle_ll_positions(int T, int k, int E, int R, const int32_t *topk_idx,
                             int32_t *pos, int32_t *src_idx, int32_t *recv_count) {
    uint32_t status = 0;
    int tpr = T / R;
    long long region = (long long)R * tpr; /* rows per expert */
    for (long long i = 0; i < (long long)E * region; ++i) src_idx[i] = -1;
    for (int i = 0; i < E * R; ++i) recv_count[i] = 0;
    for (int t = 0; t < T; ++t) {
        const int32_t *row = topk_idx + (size_t)t * k;
        int s = t / tpr;
        for (int j = 0; j < k; ++j) {
            pos[(size_t)t * k + j] = -1;
            if (!slot_is_valid(row, j, E, &status)) continue;
            int e = row[j];
            long long p = (long long)e * region + (long long)s * tpr + recv_count[e * R + s];
            recv_count[e * R + s] += 1;
            pos[(size_t)t * k + j] = (int32_t)p;
            src_idx[p] = t;
        }
    }
    return status;
}

/* Rank-deduplicated exchange: one received row per (token, destination rank)
 * instead of one per (token, expert). Reading (the pages' normal kernels send
 * a token once per rank; the row then carries which of that rank's experts
 * take it): the first valid slot of token t whose expert lives on rank d is
 * the pair's "leader" slot, and rank d's rows hold its tokens in source-token
 * order (the same stable order as the per-expert rows). */

/* rank_in_rank[t][j] = number of tokens t' < t that have a valid slot on rank
 * d(e) where e = topk_idx[t][j], if slot j is the leader of (t, d); -1 for
 * every other slot. token_rows[d] = tokens with a valid slot on rank d.
 * Returns the validation status bits and 4 if some token_rows[d] > cap_rows. */
uint32_t oracle_layout_dedup(int T, int k, int E, int R, long long cap_rows,
                             const int32_t *topk_idx, int32_t *rank_in_rank, int32_t *token_rows) {
    uint32_t status = 0;
    int experts_per_rank = E / R;
    int32_t *fill = (int32_t *)calloc((size_t)R, sizeof(int32_t));
    for (int t = 0; t < T; ++t) {
        const int32_t *row = topk_idx + (size_t)t * k;
        for (int j = 0; j < k; ++j) {
            rank_in_rank[(size_t)t * k + j] = -1;
            if (!slot_is_valid(row, j, E, &status)) continue;
            int d = row[j] / experts_per_rank;
            int leader = 1;
            for (int jj = 0; jj < j; ++jj) {
                uint32_t ignore = 0;
                if (slot_is_valid(row, jj, E, &ignore) && row[jj] / experts_per_rank == d) leader = 0;
            }
            if (!leader) continue;
            rank_in_rank[(size_t)t * k + j] = fill[d];
            fill[d] += 1;
        }
    }
    for (int d = 0; d < R; ++d) {
        token_rows[d] = fill[d];
        if ((long long)fill[d] > cap_rows) status |= ORACLE_ST_CAPACITY;
    }
    free(fill);
    return status;
}

/* Handle of the deduplicated exchange: for a leader slot (t, j) of rank d,
 * pos[t][j] = d * cap_rows + rank_in_rank[t][j] (-1 if that reaches cap_rows);
 * -1 for every other slot. src_idx[pos] = t for every kept row. */
void oracle_positions_dedup(int T, int k, int E, int R, long long cap_rows,
                            const int32_t *topk_idx, const int32_t *rank_in_rank,
                            int32_t *pos, int32_t *src_idx) {
    int experts_per_rank = E / R;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            size_t i = (size_t)t * k + j;
            int32_t r = rank_in_rank[i];
            if (r < 0 || (long long)r >= cap_rows) {
                pos[i] = -1;
                continue;
            }
            long long p = (long long)(topk_idx[i] / experts_per_rank) * cap_rows + r;
            pos[i] = (int32_t)p;
            src_idx[p] = t;
        }
    }
}

/* Deduplicated dispatch: each kept row p = pos[t][j] (leader of rank d)
 * receives token t's row once (bit copy, or FP8 with the per-group scales as
 * in oracle_dispatch), and k routing entries: for every slot j' of t,
 *   recv_topk_idx[p][j'] = e' - d * E/R  and  recv_topk_w[p][j'] = topk_w[t][j']
 * if slot j' is valid and its expert e' lives on rank d, else -1 and 0.0f.
 * recv_topk_w is skipped if it or topk_w is NULL. tokens/ntokens restricts the
 * work to a list of tokens (NULL = all T). */
void oracle_dispatch_dedup(int T, int k, int H, int E, int R, int use_fp8, const uint16_t *x,
                           const int32_t *topk_idx, const float *topk_w, const int32_t *pos,
                           const int32_t *tokens, int ntokens, void *recv_x, float *recv_scales,
                           int32_t *recv_topk_idx, float *recv_topk_w) {
    int G = H / 128;
    int experts_per_rank = E / R;
    int n = tokens ? ntokens : T;
    uint8_t *q = NULL;
    float *sc = NULL;
    if (use_fp8) {
        q = (uint8_t *)malloc((size_t)H);
        sc = (float *)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
    }
    for (int ii = 0; ii < n; ++ii) {
        int t = tokens ? tokens[ii] : ii;
        const uint16_t *xr = x + (size_t)t * H;
        const int32_t *row = topk_idx + (size_t)t * k;
        if (use_fp8) oracle_quantize_token(H, xr, q, sc);
        for (int j = 0; j < k; ++j) {
            int32_t p = pos[(size_t)t * k + j];
            if (p < 0) continue;
            int d = row[j] / experts_per_rank;
            if (use_fp8) {
                memcpy((uint8_t *)recv_x + (size_t)p * H, q, (size_t)H);
                memcpy(recv_scales + (size_t)p * G, sc, sizeof(float) * (size_t)G);
            } else {
                memcpy((uint16_t *)recv_x + (size_t)p * H, xr, sizeof(uint16_t) * (size_t)H);
            }
            for (int jj = 0; jj < k; ++jj) {
                uint32_t ignore = 0;
                int here = slot_is_valid(row, jj, E, &ignore) && row[jj] / experts_per_rank == d;
                recv_topk_idx[(size_t)p * k + jj] = here ? row[jj] - d * experts_per_rank : -1;
                if (recv_topk_w && topk_w) recv_topk_w[(size_t)p * k + jj] = here ? topk_w[(size_t)t * k + jj] : 0.0f;
            }
        }
    }
    free(q);
    free(sc);
}

/* Per-token FP8 quantization, one scale per group of 128 channels.
 * Reading (the pages say only "FP8 dispatch"): for group g,
 *   amax  = max over the group of |x|                (exact)
 *   a     = max(amax, 1e-4)                           (floor for all-zero groups)
 *   inv   = 448 / a       (one IEEE fp32 division)
 *   scale = a / 448       (one IEEE fp32 division; the value stored per group)
 *   q_i   = e4m3(x_i * inv)  (one fp32 multiply, then round-to-nearest-even,
 *                             saturating to +-448)
 * so that dequantization is q * scale and the group's largest element maps
 * to +-448. */
void oracle_quantize_token(int H, const uint16_t *x_row, uint8_t *q, float *scales) {
    int G = H / 128;
    for (int g = 0; g < G; ++g) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float v = fabsf(bf16_to_float(x_row[g * 128 + i]));
            if (v > amax) amax = v;
        }
        float a = amax > 1e-4f ? amax : 1e-4f;
        float inv = 448.0f / a;
        float scale = a / 448.0f;
        for (int i = 0; i < 128; ++i) {
            float prod = bf16_to_float(x_row[g * 128 + i]) * inv;
            q[g * 128 + i] = e4m3_from_float(prod);
        }
        scales[g] = scale;
    }
}

/* Dispatch: every kept slot (t, j) receives a copy of token t's row at
 * receive row pos[t][j]:
 *   BF16:  recv_x[p][:] = x[t][:] (bit copy, uint16 per element)
 *   FP8:   recv_x[p][:] = q(x[t]) (uint8 per element), recv_scales[p][:] = scales
 *   both:  recv_w[p] = topk_w[t][j] (if recv_w and topk_w are given)
 * tokens/ntokens restricts the work to a list of tokens (NULL = all T). */
void oracle_dispatch(int T, int k, int H, int use_fp8, const uint16_t *x,
                     const float *topk_w, const int32_t *pos,
                     const int32_t *tokens, int ntokens,
                     void *recv_x, float *recv_scales, float *recv_w) {
    int G = H / 128;
    int n = tokens ? ntokens : T;
    uint8_t *q = NULL;
    float *sc = NULL;
    if (use_fp8) {
        q = (uint8_t *)malloc((size_t)H);
        sc = (float *)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
    }
    for (int ii = 0; ii < n; ++ii) {
        int t = tokens ? tokens[ii] : ii;
        const uint16_t *xr = x + (size_t)t * H;
        if (use_fp8) oracle_quantize_token(H, xr, q, sc);
        for (int j = 0; j < k; ++j) {
            int32_t p = pos[(size_t)t * k + j];
            if (p < 0) continue;
            if (use_fp8) {
                memcpy((uint8_t *)recv_x + (size_t)p * H, q, (size_t)H);
                memcpy(recv_scales + (size_t)p * G, sc, sizeof(float) * (size_t)G);
            } else {
                memcpy((uint16_t *)recv_x + (size_t)p * H, xr, sizeof(uint16_t) * (size_t)H);
            }
            if (recv_w && topk_w) recv_w[p] = topk_w[(size_t)t * k + j];
        }
    }
    free(q);
    free(sc);
}

/* Combine (weighted gather-reduce back to source-token order):
 *   acc = +0.0f; for j = 0 .. k-1 with pos[t][j] >= 0:
 *       acc = fmaf(w[t][j], rows[pos[t][j]][i], acc)       (w = 1 if w == NULL)
 *   y[t][i] = bf16(acc)   (round to nearest even)
 * Reading: fp32 accumulation in slot order, one fused multiply-add per slot,
 * one rounding to bf16 at the end; a token with no kept slot gives +0.
 * acc (optional) receives the fp32 sums before rounding.
 * tokens/ntokens restricts the work to a list of tokens (NULL = all T); y and
 * acc are then indexed by list position. */
void oracle_combine(int T, int k, int H, const uint16_t *rows, const int32_t *pos,
                    const float *w, const int32_t *tokens, int ntokens,
                    uint16_t *y, float *acc) {
    int n = tokens ? ntokens : T;
    float *a = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    for (int ii = 0; ii < n; ++ii) {
        int t = tokens ? tokens[ii] : ii;
        for (int i = 0; i < H; ++i) a[i] = 0.0f;
        for (int j = 0; j < k; ++j) {
            int32_t p = pos[(size_t)t * k + j];
            if (p < 0) continue;
            float wt = w ? w[(size_t)t * k + j] : 1.0f;
            const uint16_t *r = rows + (size_t)p * H;
            for (int i = 0; i < H; ++i) a[i] = fmaf(wt, bf16_to_float(r[i]), a[i]);
        }
        for (int i = 0; i < H; ++i) {
            y[(size_t)ii * H + i] = bf16_from_float(a[i]);
            if (acc) acc[(size_t)ii * H + i] = a[i];
        }
    }
    free(a);
}

/* Expert-side pre-reduction of the rank-deduplicated rows. Reading (the
 * pages' normal kernels send a token once per destination rank, and the
 * guide's combine brings the experts' outputs back to the token's rank):
 * rank d holds one received row per token it serves; each of its experts
 * that the token chose produces an output for that row, and the rank sums
 * those outputs with the row's routing weights, so that combine sends one
 * row back per (token, rank). Layout of the expert outputs: for received row
 * p and slot j, expert_out[p][j][:] (bf16) is the output of the row's slot-j
 * expert; only slots whose routing entry recv_topk_idx[p][j] is >= 0 are
 * read. For every used row p of rank d (p - d*cap_rows below both
 * token_rows[d] and cap_rows), channel i:
 *   sum = +0.0f; for j = 0 .. k-1 with recv_topk_idx[p][j] >= 0:
 *       sum = fmaf(weight, expert_out[p][j][i], sum)
 *                     (weight = recv_topk_w[p][j], or 1 if recv_topk_w is NULL)
 *   reduced[p][i] = bf16(sum)   (round to nearest even)
 * the arithmetic of oracle_combine (fp32, one fused multiply-add per slot in
 * slot order, one rounding). Rows that are not used are left untouched.
 * Only rows [row_lo, row_hi) are computed; every array holds exactly those
 * rows (row p at index p - row_lo). sums (optional) receives the fp32 sums. */
void oracle_prereduce(int R, long long cap_rows, int k, int H, long long row_lo, long long row_hi,
                      const uint16_t *expert_out, const int32_t *recv_topk_idx,
                      const float *recv_topk_w, const int32_t *token_rows,
                      uint16_t *reduced, float *sums) {
    float *s = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    for (long long p = row_lo; p < row_hi; ++p) {
        long long d = p / cap_rows;
        long long local = p - d * cap_rows;
        if (d >= R || local >= (long long)token_rows[d]) continue; /* not a used row */
        long long r = p - row_lo;
        for (int i = 0; i < H; ++i) s[i] = 0.0f;
        for (int slot = 0; slot < k; ++slot) {
            if (recv_topk_idx[r * k + slot] < 0) continue;
            float weight = recv_topk_w ? recv_topk_w[r * k + slot] : 1.0f;
            const uint16_t *out = expert_out + ((size_t)r * k + slot) * (size_t)H;
            for (int i = 0; i < H; ++i) s[i] = fmaf(weight, bf16_to_float(out[i]), s[i]);
        }
        for (int i = 0; i < H; ++i) {
            reduced[(size_t)r * H + i] = bf16_from_float(s[i]);
            if (sums) sums[(size_t)r * H + i] = s[i];
        }
    }
    free(s);
}

/* combine_backward: the gradient of combined_x is sent along the same routes
 * as dispatch (a bf16 dispatch of grad_y reusing the forward handle):
 *   grad_rows[pos[t][j]][:] = grad_y[t][:] for every kept slot.
 * (dispatch_backward is oracle_combine applied to grad_rows.) */
void oracle_combine_backward(int T, int k, int H, const uint16_t *grad_y,
                             const int32_t *pos, uint16_t *grad_rows) {
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t p = pos[(size_t)t * k + j];
            if (p < 0) continue;
            memcpy(grad_rows + (size_t)p * H, grad_y + (size_t)t * H, sizeof(uint16_t) * (size_t)H);
        }
    }
}
