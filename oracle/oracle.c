/*
 * Float64 CPU oracle for relative-bias grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's compute path may link,
 * load or call this file. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header or constant
 * with the HIP kernels.
 *
 * What it computes is the plain definition, with no tiling, blocking or
 * online softmax:
 *
 *   For query row t of sequence b (absolute position i) and query head h,
 *   with KV head g = h / (Hq / Hkv):
 *     visible keys  j with  j <= i  and, when W > 0,  i - j < W
 *     score x_j  =  scale * sum_d q[t,h,d] * K_b[j,g,d]  +  bias(i - j)
 *     bias(d)    =  rel[t,h,d]  for 0 <= d < R,  0 for d >= R
 *     out[t,h,:] =  sum_j softmax(x)_j * V_b[j,g,:]
 *     lse[t,h]   =  log sum_j exp(x_j)
 *   Optional gated-attention outputs (sink, gate may each be NULL):
 *     with a sink logit s = sink[t,h] the softmax set is {x_j} plus s, whose
 *     value vector is zero:  out = sum_j exp(x_j) V_j / (sum_j exp(x_j) + exp(s)),
 *     lse = log(sum_j exp(x_j) + exp(s));
 *     with a gate logit a = gate[t,h] the output is scaled by 1 / (1 + exp(-a)).
 *
 * Sources (the pages, not code):
 *  - "Inkling-Small on Gaudi 2", section "Why it needed a port": the relative
 *    logit is a per-query, per-head, per-distance term indexed by i - j and
 *    added to the attention logit.
 *  - same page, "What was built": GQA with 32 query / 8 KV heads of size 128;
 *    local layers use a 512-token window with relative extent 512, global
 *    layers have no window and extent 1024.
 *  - same page, "Attention with a relative bias": rel is computed per query
 *    token from the R branch for the tokens of the current call; chunked
 *    prefill attends to the cached context plus the chunk itself; key
 *    positions are block ordinals times the block size plus the slot.
 *  - same page, "Decode window": the window is cut at exactly W keys,
 *    counting the query's own key (reading taken: visible iff 0 <= i-j < W).
 *  - "Inkling on Two DGX Sparks ...", section "Wall 1": head_dim 128 with
 *    v_head_dim 64 (value head size may differ from the query/key size), and
 *    validation of every path against a float64 reference.
 *  - The pages do not say what the bias is for distances at or beyond the
 *    relative extent; this oracle uses 0 there (the reading the library
 *    documents as well).
 *  - "Inkling 2 Small on vLLM: Day-0 Support", section on the model
 *    architecture (table row on the attention output, and the paragraph on
 *    the Inkling backbone and recent advances): each head's output gets a
 *    sigmoid gate, paired with a per-token attention sink. No formula is
 *    given; the reading above (a per-(token, head) sink logit in the softmax
 *    normaliser with a zero value, and a per-(token, head) sigmoid factor on
 *    the output) is this oracle's and the library's.
 *
 * Layouts (all contiguous, row-major, float64):
 *   q    [total_q, Hq, dqk]     rows of all sequences packed; sequence b owns
 *                               rows [q_start_b, q_start_b + q_len_b)
 *   k    [total_kv, Hkv, dqk]   un-paged keys; sequence b owns rows
 *                               [kv_start_b, kv_start_b + seq_len_b)
 *   v    [total_kv, Hkv, dv]
 *   rel  [total_q, Hq, R]
 *   out  [total_q, Hq, dv]
 *   lse  [total_q, Hq]          (may be NULL)
 *   sink, gate [total_q, Hq]    (each may be NULL)
 * The query rows of sequence b are its last q_len_b positions:
 *   i = seq_len_b - q_len_b + (t - q_start_b).
 *
 * rows/n_rows: if rows != NULL only those global query rows are computed (the
 * other rows of out/lse are left untouched); used to sample large inputs.
 *
 * Return 0 on success, -1 on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static int find_seq(const int64_t* q_start, int64_t batch, int64_t t) {
    /* last b with q_start[b] <= t (sequences with q_len 0 are skipped) */
    int64_t lo = 0, hi = batch - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) / 2;
        if (q_start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return (int)lo;
}

int rba_oracle_attend(int64_t batch, const int64_t* q_lens, const int64_t* seq_lens,
                      int64_t Hq, int64_t Hkv, int64_t dqk, int64_t dv,
                      int64_t R, int64_t W, double scale,
                      const double* q, const double* k, const double* v,
                      const double* rel, const double* sink, const double* gate,
                      const int64_t* rows, int64_t n_rows,
                      double* out, double* lse) {
    if (batch <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || dqk <= 0 || dv <= 0 ||
        R < 1 || W < 0)
        return -1;
    int64_t* q_start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(batch + 1));
    int64_t* kv_start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(batch + 1));
    if (!q_start || !kv_start) { free(q_start); free(kv_start); return -1; }
    q_start[0] = 0; kv_start[0] = 0;
    for (int64_t b = 0; b < batch; ++b) {
        if (q_lens[b] < 0 || q_lens[b] > seq_lens[b]) { free(q_start); free(kv_start); return -1; }
        q_start[b + 1] = q_start[b] + q_lens[b];
        kv_start[b + 1] = kv_start[b] + seq_lens[b];
    }
    const int64_t total_q = q_start[batch];
    const int64_t G = Hq / Hkv;
    const int64_t n_work = (rows ? n_rows : total_q) * Hq;

#pragma omp parallel
    {
        /* one scratch vector of scores per thread, sized for the longest sequence */
        int64_t max_len = 0;
        for (int64_t b = 0; b < batch; ++b) if (seq_lens[b] > max_len) max_len = seq_lens[b];
        double* x = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));

#pragma omp for schedule(dynamic, 16)
        for (int64_t w = 0; w < n_work; ++w) {
            const int64_t t = rows ? rows[w / Hq] : w / Hq;
            const int64_t h = w % Hq;
            if (t < 0 || t >= total_q) continue;
            /* owner of row t: the last sequence whose first row is <= t */
            const int b = find_seq(q_start, batch, t);
            const int64_t i = seq_lens[b] - q_lens[b] + (t - q_start[b]);
            const int64_t g = h / G;
            const int64_t lo = (W == 0) ? 0 : (i - W + 1 > 0 ? i - W + 1 : 0);
            const double* qr = q + (t * Hq + h) * dqk;
            const double* relr = rel + (t * Hq + h) * R;

            /* scores of the visible keys j = lo..i */
            double m = -INFINITY;
            for (int64_t j = lo; j <= i; ++j) {
                const double* kr = k + ((kv_start[b] + j) * Hkv + g) * dqk;
                double s = 0.0;
                for (int64_t d = 0; d < dqk; ++d) s += qr[d] * kr[d];
                const int64_t dist = i - j;
                const double bias = dist < R ? relr[dist] : 0.0;
                x[j - lo] = scale * s + bias;
                if (x[j - lo] > m) m = x[j - lo];
            }
            /* the sink logit joins the softmax set (its value is zero) */
            const double sk = sink ? sink[t * Hq + h] : -INFINITY;
            if (sk > m) m = sk;
            /* softmax weights and the weighted sum of values */
            double l = sink ? exp(sk - m) : 0.0;
            for (int64_t j = lo; j <= i; ++j) {
                x[j - lo] = exp(x[j - lo] - m);
                l += x[j - lo];
            }
            double* o = out + (t * Hq + h) * dv;
            for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
            for (int64_t j = lo; j <= i; ++j) {
                const double p = x[j - lo] / l;
                const double* vr = v + ((kv_start[b] + j) * Hkv + g) * dv;
                for (int64_t c = 0; c < dv; ++c) o[c] += p * vr[c];
            }
            if (gate) {
                const double f = 1.0 / (1.0 + exp(-gate[t * Hq + h]));
                for (int64_t c = 0; c < dv; ++c) o[c] *= f;
            }
            if (lse) lse[t * Hq + h] = m + log(l);
        }
        free(x);
    }
    free(q_start);
    free(kv_start);
    return 0;
}
