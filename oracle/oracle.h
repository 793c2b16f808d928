/*
 * oracle.h -- plain fp64 CPU reference for exact attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this library; only the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library.
 *
 * What it computes is the textbook definition of scaled-dot-product
 * attention, which the pages say FlashAttention reproduces exactly:
 *   - "推理加速" interview notes, section FlashAttention ("它到底优化了什么"):
 *     the method is not an approximation and stays mathematically equal to
 *     standard attention;
 *   - chenyy20.com "抱infra脚", section Flash Attention 基本原理 / 核心技术:
 *     the naive workflow writes S = QK^T out, forms P = softmax(S), then O = PV.
 * The oracle follows that naive workflow: S and P are materialised in full
 * for every (batch, query head), in double precision.
 *
 * Tensor layouts (all row-major, contiguous, D innermost; values are the
 * exact bf16 or fp32 inputs widened to float):
 *   q   [B, Sq, Hq,  D]     k, v [B, Sk, Hkv, D]
 *   o   [B, Sq, Hq,  D]     lse  [B, Hq, Sq]          (double)
 * Query head h reads key/value head h / (Hq / Hkv) (consecutive grouping).
 * Causal visibility is bottom-right aligned: key j is visible to query i iff
 * j <= i + (Sk - Sq).  A query with no visible key gets O = 0, lse = -inf.
 * lse is the natural-log log-sum-exp of the scaled scores of the visible keys.
 *
 * All functions return 0 on success and a negative value on bad arguments
 * or allocation failure.
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Full attention, all rows.  nthreads <= 0 uses the OpenMP default. */
int oracle_attention(const float *q, const float *k, const float *v,
                     double *o, double *lse,
                     long B, long Sq, long Sk, long Hq, long Hkv, long D,
                     int causal, double scale, int nthreads);

/* The same definition evaluated for nrows selected (b, h, i) rows only.
 * o is [nrows, D], lse is [nrows]. */
int oracle_attention_rows(const float *q, const float *k, const float *v,
                          long B, long Sq, long Sk, long Hq, long Hkv, long D,
                          int causal, double scale,
                          const long *row_b, const long *row_h, const long *row_i,
                          long nrows, double *o, double *lse, int nthreads);

/* Materialised score and probability matrices of one (b, hq): S and P are
 * [Sq, Sk]; masked entries hold S = -inf and P = 0. */
int oracle_scores_probs(const float *q, const float *k,
                        long B, long Sq, long Sk, long Hq, long Hkv, long D,
                        int causal, double scale, long b, long hq,
                        double *S, double *P);

/* Single-token decode on the logical (unpaged) per-sequence keys/values:
 *   q [B, Hq, D]; sequence b's keys are k_log[seq_off[b] .. seq_off[b] +
 *   ctx[b]) with rows of [Hkv, D]; all ctx[b] keys are visible.
 *   o [B, Hq, D], lse [B, Hq]. */
int oracle_decode(const float *q, const float *k_log, const float *v_log,
                  const long *seq_off, const long *ctx,
                  long B, long Hq, long Hkv, long D, double scale,
                  double *o, double *lse, int nthreads);

/* Merge n partial results of the same query row, each computed over a
 * disjoint subset of the keys and normalised within that subset
 * (o_parts [n, D], lse_parts [n]; an empty subset has lse = -inf), into the
 * result over the union.  This is the log-sum-exp merge that Flash-Decoding
 * applies to its per-chunk partial outputs ("GPU Kernel 调度：大模型推理的拐点
 * 2026", paragraphs on Flash Decoding and on its reduce-kernel cost). */
int oracle_lse_combine(const double *o_parts, const double *lse_parts, long n,
                       long D, double *o, double *lse);

#ifdef __cplusplus
}
#endif

#endif
