/*
 * sa_oracle.c -- plain, slow CPU reference for the sparse flash-attention forward paths.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or loads this file; only
 * the tests, the package smoke check and the benchmark's CPU-baseline leg do.  It shares no code,
 * header, table or constant with the HIP kernels: it reads the same bf16 bit patterns the GPU reads
 * (upcast exactly to double) and accumulates everything in double precision with host libm.
 *
 * Every function takes Q [B,Sq,Hq,D], K/V [B,Sk,Hkv,D] as contiguous bf16 bit patterns (uint16) and
 * works on a list of independent "units" (one unit = one (batch, query head, query tile) triple);
 * results are written per unit in unit order.  Units are spread over OpenMP threads; the arithmetic
 * of one unit is a plain sequential loop in the order the method states.
 *
 * Method sources (cited by page title and section):
 *   [MO-diff]  Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion Models" README:
 *              introduction (skip KV tiles whose scores are negligible during FlashAttention),
 *              "Threshold Modes" table (kernel uses log2(lambda); calibrated lambda =
 *              a*exp(b*target_sparsity)/seq_k).
 *   [MO-llm]   Model-Optimizer "Attention Sparsity for HuggingFace Models": method list
 *              (skip-softmax skips tiles with negligible contribution; N:M keeps the top-N of every
 *              M consecutive keys and sets the rest to -inf before softmax), "N:M Sparse Softmax"
 *              section (M=4 with N=1..3, M=8 with N=1..7, dense sink and recent tokens, prefill only).
 *   [FI-proxy] FlashInfer block-sparse proxy description (quoted in the TensorRT-LLM "add VisualGen
 *              SOL sparse attention" PR): "Description" (exact blocks + arithmetic-mean K and
 *              summed V per omitted block, denominator corrected by the represented token mass
 *              including the final partial block) and "Bitmask format" (packed UInt32 per
 *              (batch, KV head, Q block), padding bits ignored).
 *
 * Readings where the pages are silent are listed beside each function; they are the same readings
 * the kernel documentation states.  Parity status of each function is given in its comment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element (b, s, h, e) of a contiguous [B, S, H, D] bf16 tensor, as a double. */
static double at(const uint16_t* x, int S, int H, int D, int b, int s, int h, int e) {
    return bf16_value(x[(((int64_t)b * S + s) * H + h) * D + e]);
}

static double dot_qk(const uint16_t* q, const uint16_t* k, int Sq, int Sk, int Hq, int Hkv, int D,
                     int b, int r, int hq, int key, int hk) {
    double acc = 0.0;
    for (int e = 0; e < D; ++e)
        acc += at(q, Sq, Hq, D, b, r, hq, e) * at(k, Sk, Hkv, D, b, key, hk, e);
    return acc;
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------------------
 * Skip-softmax (BLASST-style) forward.  [MO-diff] introduction + "Threshold Modes"; [MO-llm]
 * method list.  An approximation, so the steps follow the method in order:
 *
 *   FlashAttention over KV tiles in ascending order with running max m, running sum l and
 *   accumulator acc per query row.  For each visited tile j, the log2-domain logits
 *   t = scale*log2(e)*q.k give the tile row maxima M_j[r].  The tile is negligible, and skipped
 *   with its softmax and its P.V, when every valid row satisfies M_j[r] < m[r] + log2(lambda).
 *   A skipped tile leaves (m, l, acc) untouched; a kept tile takes the usual online-softmax update.
 *
 * Readings: negligible means "ratio to the running max of the tiles kept so far is below lambda";
 * the test is strict, so lambda = 0 (log2 = -inf) never skips; the whole Br x Bc tile is skipped
 * only if all of its valid rows are negligible; rows >= Sq are not part of the tile; a row with
 * every key of the tile masked has M = -inf; causal masking is top-left (key <= query); a tile is
 * visited when it holds at least one unmasked (row, key) pair.
 *
 * mode 0: independent decisions in double.
 * mode 1: replay -- M_j[r] is taken from rowmax_in (fp32, log2 domain, as the GPU used it) and the
 *         test is done in fp32 as  M < (float)(m32 + L32), L32 = (float)log2((double)lambda),
 *         with m32 the fp32 running max of the replayed maxima.  Arithmetic (l, acc) stays double.
 * mode 2: decisions forced from state_in (0 kept, 1 skipped); used to compare outputs on the
 *         kept-tile set the GPU chose.
 *
 * Outputs per unit u: o_out[u][Br][D] (double), lse_out[u][Br] (natural log), state_out[u][nKT]
 * (0 kept, 1 skipped, 2 not visited), rowmax_out[u][nKT][Br] (double, log2 domain; -inf where the
 * row has no unmasked key in the tile or the tile is not visited).  Rows >= Sq are written as 0.
 * ----------------------------------------------------------------------------------------------*/
int oracle_skip_softmax(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int Br, int Bc,
                        double scale, double lambda, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, int mode, const float* rowmax_in, const uint8_t* state_in,
                        const int64_t* units, int64_t n_units, double* o_out, double* lse_out,
                        uint8_t* state_out, double* rowmax_out) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Sq < 1 || Sk < 1 || D < 1 || Br < 1 || Bc < 1)
        return 1;
    if (causal && Sq != Sk) return 1;
    if (!(lambda >= 0.0) || isinf(lambda)) return 1;
    const int nQT = (Sq + Br - 1) / Br, nKT = (Sk + Bc - 1) / Bc;
    const int group = Hq / Hkv;
    const double c = scale * M_LOG2E;
    const double L = (lambda == 0.0) ? -INFINITY : log2(lambda);
    const float L32 = (lambda == 0.0) ? -INFINITY : (float)log2((double)(float)lambda);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_units; ++u) {
        const int64_t unit = units ? units[u] : u;
        if (unit < 0 || unit >= (int64_t)B * Hq * nQT) { bad = 1; continue; }
        const int i = (int)(unit % nQT);
        const int hq = (int)((unit / nQT) % Hq);
        const int b = (int)(unit / ((int64_t)nQT * Hq));
        const int hk = hq / group;
        const int r0 = i * Br, r1 = (r0 + Br < Sq) ? r0 + Br : Sq, nr = r1 - r0;

        double* m = malloc(sizeof(double) * Br);
        double* l = malloc(sizeof(double) * Br);
        float* m32 = malloc(sizeof(float) * Br);
        double* acc = calloc((size_t)Br * D, sizeof(double));
        double* t = malloc(sizeof(double) * Br * Bc);
        double* M = malloc(sizeof(double) * Br);
        for (int r = 0; r < Br; ++r) { m[r] = -INFINITY; l[r] = 0.0; m32[r] = -INFINITY; }

        for (int j = 0; j < nKT; ++j) {
            const int k0 = j * Bc, k1 = (k0 + Bc < Sk) ? k0 + Bc : Sk;
            uint8_t* st = &state_out[u * nKT + j];
            double* rm = &rowmax_out[(u * nKT + j) * Br];
            for (int r = 0; r < Br; ++r) rm[r] = -INFINITY;
            /* visited: at least one unmasked pair; causal top-left means key <= row */
            int visited = causal ? (k0 <= r1 - 1) : 1;
            if (!visited) { *st = 2; continue; }

            /* logits of the tile (log2 domain) and their row maxima */
            for (int rr = 0; rr < nr; ++rr) {
                const int r = r0 + rr;
                M[rr] = -INFINITY;
                for (int kk = k0; kk < k1; ++kk) {
                    double tv = -INFINITY;
                    if (!causal || kk <= r)
                        tv = c * dot_qk(q, k, Sq, Sk, Hq, Hkv, D, b, r, hq, kk, hk);
                    t[rr * Bc + (kk - k0)] = tv;
                    if (tv > M[rr]) M[rr] = tv;
                }
                rm[rr] = M[rr];
            }

            /* decision: skip iff every valid row is negligible against the running max */
            int skip;
            if (mode == 2) {
                skip = state_in[unit * nKT + j] == 1;
            } else if (mode == 1) {
                const float* Min = &rowmax_in[(unit * nKT + j) * Br];
                skip = 1;
                for (int rr = 0; rr < nr; ++rr)
                    if (!(Min[rr] < (float)(m32[rr] + L32))) { skip = 0; break; }
            } else {
                skip = 1;
                for (int rr = 0; rr < nr; ++rr)
                    if (!(M[rr] < m[rr] + L)) { skip = 0; break; }
            }
            *st = (uint8_t)skip;
            if (skip) continue;

            /* online-softmax update with the kept tile */
            for (int rr = 0; rr < nr; ++rr) {
                if (mode == 1) {
                    const float Mf = rowmax_in[(unit * nKT + j) * Br + rr];
                    if (Mf > m32[rr]) m32[rr] = Mf;
                }
                const double m_new = (M[rr] > m[rr]) ? M[rr] : m[rr];
                if (m_new == -INFINITY) continue; /* no unmasked key seen yet in this row */
                const double alpha = (m[rr] == -INFINITY) ? 0.0 : exp2(m[rr] - m_new);
                l[rr] *= alpha;
                for (int e = 0; e < D; ++e) acc[rr * D + e] *= alpha;
                for (int kk = k0; kk < k1; ++kk) {
                    const double tv = t[rr * Bc + (kk - k0)];
                    if (tv == -INFINITY) continue;
                    const double p = exp2(tv - m_new);
                    l[rr] += p;
                    for (int e = 0; e < D; ++e)
                        acc[rr * D + e] += p * at(v, Sk, Hkv, D, b, kk, hk, e);
                }
                m[rr] = m_new;
            }
        }
        for (int rr = 0; rr < Br; ++rr) {
            double* o = &o_out[(u * Br + rr) * D];
            if (rr >= nr || l[rr] == 0.0) {
                for (int e = 0; e < D; ++e) o[e] = 0.0;
                lse_out[u * Br + rr] = (rr >= nr) ? 0.0 : -INFINITY;
                continue;
            }
            for (int e = 0; e < D; ++e) o[e] = acc[rr * D + e] / l[rr];
            lse_out[u * Br + rr] = (m[rr] + log2(l[rr])) * M_LN2;
        }
        free(m); free(l); free(m32); free(acc); free(t); free(M);
    }
    return bad;
}

/* ------------------------------------------------------------------------------------------------
 * Skip-softmax decisions replayed from given tile maxima, without the attention arithmetic.
 * [MO-diff] introduction + "Threshold Modes".  This is the decision chain of oracle_skip_softmax in
 * mode 1 on its own (no logits, no softmax), so that a whole full-size run can be replayed:
 *
 *   for each unit (b, hq, query tile i of Br rows; valid rows r0 .. r1-1) and each key tile j of Bc
 *   keys in ascending order, visited when it holds an unmasked pair (causal: j*Bc <= r1-1):
 *     skip(j) = every valid row rr has  M_j[rr] < (float)(m32[rr] + L32),
 *               L32 = (float)log2((double)(float)lambda), -inf for lambda == 0;
 *     a kept tile raises m32[rr] to max(m32[rr], M_j[rr]); a skipped tile changes nothing.
 *
 * The comparison and the running max are fp32, as in mode 1 of oracle_skip_softmax.
 * rowmax holds the maxima of the listed units only, compact: [n_units][nKT][Br] (fp32, log2
 * domain; entries of rows >= Sq and of unvisited tiles are not read).  state_out [n_units][nKT]:
 * 0 kept, 1 skipped, 2 not visited.  Units are linear (b*Hq + hq)*nQT + i; NULL means all.
 * ----------------------------------------------------------------------------------------------*/
int oracle_skip_replay(int B, int Hq, int Sq, int Sk, int causal, int Br, int Bc, double lambda,
                       const int64_t* units, int64_t n_units, const float* rowmax,
                       uint8_t* state_out) {
    if (B < 1 || Hq < 1 || Sq < 1 || Sk < 1 || Br < 1 || Bc < 1) return 1;
    if (causal && Sq != Sk) return 1;
    if (!(lambda >= 0.0) || isinf(lambda)) return 1;
    const int nQT = (Sq + Br - 1) / Br, nKT = (Sk + Bc - 1) / Bc;
    const float L32 = (lambda == 0.0) ? -INFINITY : (float)log2((double)(float)lambda);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t u = 0; u < n_units; ++u) {
        const int64_t unit = units ? units[u] : u;
        if (unit < 0 || unit >= (int64_t)B * Hq * nQT) { bad = 1; continue; }
        const int i = (int)(unit % nQT);
        const int r0 = i * Br, r1 = (r0 + Br < Sq) ? r0 + Br : Sq, nr = r1 - r0;
        float* m32 = malloc(sizeof(float) * Br);
        for (int rr = 0; rr < Br; ++rr) m32[rr] = -INFINITY;
        for (int j = 0; j < nKT; ++j) {
            uint8_t* st = &state_out[u * nKT + j];
            const int visited = causal ? (j * Bc <= r1 - 1) : 1;
            if (!visited) { *st = 2; continue; }
            const float* Min = &rowmax[((size_t)u * nKT + j) * Br];
            int skip = 1;
            for (int rr = 0; rr < nr; ++rr)
                if (!(Min[rr] < (float)(m32[rr] + L32))) { skip = 0; break; }
            *st = (uint8_t)skip;
            if (skip) continue;
            for (int rr = 0; rr < nr; ++rr)
                if (Min[rr] > m32[rr]) m32[rr] = Min[rr];
        }
        free(m32);
    }
    return bad;
}

/* N:M keep flags of one query row r over all Sk keys (the definition below, under oracle_nm_softmax):
 * x[kk] holds the ranking scores (-inf where not allowed); keep[kk] receives allowed and (dense or
 * rank < N). */
static void nm_keep_row(int r, int Sk, int causal, int N, int Mg, int sink, int recent,
                        const double* x, unsigned char* keep) {
    for (int kk = 0; kk < Sk; ++kk) {
        const int allowed = !causal || kk <= r;
        const int dense = allowed && (kk < sink || (r - kk >= 0 && r - kk < recent));
        const int g0 = (kk / Mg) * Mg;
        const int g1 = (g0 + Mg < Sk) ? g0 + Mg : Sk;
        int rank = 0;
        for (int k2 = g0; k2 < g1; ++k2)
            if (x[k2] > x[kk] || (x[k2] == x[kk] && k2 < kk)) ++rank;
        keep[kk] = (unsigned char)(allowed && (dense || rank < N));
    }
}

/* ------------------------------------------------------------------------------------------------
 * N:M sparse softmax forward.  [MO-llm] method list and "N:M Sparse Softmax".  The result is its
 * own definition, so this is the definition written out:
 *
 *   allowed(r,k) = k < Sk and (not causal or k <= r)
 *   dense(r,k)   = allowed and (k < sink or 0 <= r-k < recent)
 *   group(k)     = the M consecutive keys [floor(k/M)*M, +M) clipped to Sk
 *   x(r,k)       = q_r . k_k if allowed else -inf          (ranking on raw scores)
 *   rank(r,k)    = #{k' in group(k): x(k') > x(k) or (x(k') == x(k) and k' < k)}
 *   keep(r,k)    = allowed and (dense or rank < N)
 *   O[r]         = softmax over kept keys of scale*x, applied to V   (two passes, double)
 *
 * Readings: groups are aligned to key 0; ranking is among all members of the group, sink/recent
 * and masked entries included (masked entries are -inf and rank last); ties go to the lower key
 * index; "recent" is the R keys at or before the query (also non-causally); a partial last group
 * ranks only its valid keys.
 *
 * mode 0: scores in double.  mode 1: scores taken from scores_in [B,Hq,Sq,Sk] (fp32, as the GPU
 * ranked them) for the keep decision; the output arithmetic stays double.  mode 2: keep bits forced
 * from keep_in [B,Hq,Sq,W].  keep_out is [n_units][Br][W] with W = ceil(Sk/32), bit k&31 of word
 * k>>5 (LSB first); padding bits 0.
 * ----------------------------------------------------------------------------------------------*/
int oracle_nm_softmax(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int Br,
                      double scale, int N, int Mg, int sink, int recent, const uint16_t* q,
                      const uint16_t* k, const uint16_t* v, int mode, const float* scores_in,
                      const uint32_t* keep_in, const int64_t* units, int64_t n_units,
                      double* o_out, double* lse_out, uint32_t* keep_out) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Sq < 1 || Sk < 1 || D < 1 || Br < 1) return 1;
    if (causal && Sq != Sk) return 1;
    if (Mg < 1 || N < 1 || N > Mg || sink < 0 || recent < 0) return 1;
    const int nQT = (Sq + Br - 1) / Br, W = (Sk + 31) / 32, group = Hq / Hkv;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_units; ++u) {
        const int64_t unit = units ? units[u] : u;
        if (unit < 0 || unit >= (int64_t)B * Hq * nQT) { bad = 1; continue; }
        const int i = (int)(unit % nQT);
        const int hq = (int)((unit / nQT) % Hq);
        const int b = (int)(unit / ((int64_t)nQT * Hq));
        const int hk = hq / group;
        double* x = malloc(sizeof(double) * Sk);
        unsigned char* keep = malloc(Sk);
        double* num = malloc(sizeof(double) * D);
        for (int rr = 0; rr < Br; ++rr) {
            const int r = i * Br + rr;
            uint32_t* kw = &keep_out[(u * Br + rr) * W];
            for (int w = 0; w < W; ++w) kw[w] = 0u;
            double* o = &o_out[(u * Br + rr) * D];
            if (r >= Sq) {
                for (int e = 0; e < D; ++e) o[e] = 0.0;
                lse_out[u * Br + rr] = 0.0;
                continue;
            }
            const int64_t row = (((int64_t)b * Hq + hq) * Sq + r);
            for (int kk = 0; kk < Sk; ++kk) {
                const int allowed = !causal || kk <= r;
                if (!allowed) x[kk] = -INFINITY;
                else if (mode == 1) x[kk] = (double)scores_in[row * Sk + kk];
                else x[kk] = dot_qk(q, k, Sq, Sk, Hq, Hkv, D, b, r, hq, kk, hk);
            }
            if (mode == 2) {
                for (int kk = 0; kk < Sk; ++kk)
                    keep[kk] = (unsigned char)((keep_in[row * W + (kk >> 5)] >> (kk & 31)) & 1u);
            } else {
                nm_keep_row(r, Sk, causal, N, Mg, sink, recent, x, keep);
            }
            for (int kk = 0; kk < Sk; ++kk)
                if (keep[kk]) kw[kk >> 5] |= 1u << (kk & 31);

            /* two-pass softmax over the kept keys, scores recomputed in double */
            double mu = -INFINITY;
            for (int kk = 0; kk < Sk; ++kk) {
                if (!keep[kk]) continue;
                const double s = scale * dot_qk(q, k, Sq, Sk, Hq, Hkv, D, b, r, hq, kk, hk);
                x[kk] = s;
                if (s > mu) mu = s;
            }
            double den = 0.0;
            for (int e = 0; e < D; ++e) num[e] = 0.0;
            for (int kk = 0; kk < Sk; ++kk) {
                if (!keep[kk]) continue;
                const double p = exp(x[kk] - mu);
                den += p;
                for (int e = 0; e < D; ++e) num[e] += p * at(v, Sk, Hkv, D, b, kk, hk, e);
            }
            if (den == 0.0) {
                for (int e = 0; e < D; ++e) o[e] = 0.0;
                lse_out[u * Br + rr] = -INFINITY;
                continue;
            }
            for (int e = 0; e < D; ++e) o[e] = num[e] / den;
            lse_out[u * Br + rr] = mu + log(den);
        }
        free(x); free(keep); free(num);
    }
    return bad;
}

/* ------------------------------------------------------------------------------------------------
 * N:M keep bits replayed from given scores, without the attention arithmetic.  [MO-llm] "N:M
 * Sparse Softmax": the keep rule of oracle_nm_softmax (its definition, nm_keep_row) applied to
 * score rows taken as given, as mode 1 of oracle_nm_softmax does, with no output computed.
 *
 *   row_pos[i]   the query position r of score row i (0 <= r < Sq)
 *   scores       [n_rows][Sk] fp32 raw scores q.k (entries of masked keys are not read: a key
 *                with causal && k > r is -inf)
 *   keep_out     [n_rows][W], W = ceil(Sk/32): bit k&31 of word k>>5 (LSB first); padding 0.
 * ----------------------------------------------------------------------------------------------*/
int oracle_nm_keep_replay(int Sq, int Sk, int causal, int N, int Mg, int sink, int recent,
                          const int32_t* row_pos, int64_t n_rows, const float* scores,
                          uint32_t* keep_out) {
    if (Sq < 1 || Sk < 1 || Mg < 1 || N < 1 || N > Mg || sink < 0 || recent < 0) return 1;
    if (causal && Sq != Sk) return 1;
    const int W = (Sk + 31) / 32;
    int bad = 0;

#pragma omp parallel
    {
        double* x = malloc(sizeof(double) * Sk);
        unsigned char* keep = malloc(Sk);
#pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < n_rows; ++i) {
            const int r = row_pos[i];
            uint32_t* kw = &keep_out[i * W];
            for (int w = 0; w < W; ++w) kw[w] = 0u;
            if (r < 0 || r >= Sq) { bad = 1; continue; }
            for (int kk = 0; kk < Sk; ++kk) {
                const int allowed = !causal || kk <= r;
                x[kk] = allowed ? (double)scores[i * Sk + kk] : -INFINITY;
            }
            nm_keep_row(r, Sk, causal, N, Mg, sink, recent, x, keep);
            for (int kk = 0; kk < Sk; ++kk)
                if (keep[kk]) kw[kk >> 5] |= 1u << (kk & 31);
        }
        free(x);
        free(keep);
    }
    return bad;
}

/* ------------------------------------------------------------------------------------------------
 * Skip-softmax combined with N:M sparse softmax.  [MO-llm] "Custom Configuration" and the example
 * script's skip_softmax_calib_sparse24 configuration (calibrated skip-softmax together with 2:4
 * sparse softmax in one attention), with the two methods as above.  Reading: the N:M rule first
 * fixes which keys of each query row may enter the softmax (the others become -inf); the
 * skip-softmax loop then runs over the key tiles of those masked logits.  So, in order:
 *
 *   keep(r,k)  as in oracle_nm_softmax (ranking on raw scores q.k)
 *   for each visited tile j in ascending order:
 *     t[r][k] = c*q.k if keep(r,k) else -inf;  M_j[r] = max_k t[r][k]
 *     skip iff every valid row has M_j[r] < m[r] + log2(lambda)   (m: running max of kept tiles)
 *     kept tiles: the online-softmax update over their finite t.
 *
 * The group maximum always survives top-N (N >= 1), so M_j equals the tile max of the unmasked
 * logits and the skip decisions equal those of skip-softmax alone.
 *
 * mode 0: double throughout.  mode 1 (replay): skip decisions from rowmax_in (fp32) as in
 * oracle_skip_softmax and N:M ranks from scores_in [B,Hq,Sq,Sk] (fp32).  mode 2: tile states from
 * state_in and keep bits from keep_in [B,Hq,Sq,W].  Outputs: o_out, lse_out, state_out and
 * rowmax_out as oracle_skip_softmax (rowmax over the kept keys), keep_out [n_units][Br][W] as
 * oracle_nm_softmax (the N:M keep bits, whatever the tile decision).
 * ----------------------------------------------------------------------------------------------*/
int oracle_skip_nm_softmax(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int Br,
                           int Bc, double scale, double lambda, int N, int Mg, int sink, int recent,
                           const uint16_t* q, const uint16_t* k, const uint16_t* v, int mode,
                           const float* rowmax_in, const uint8_t* state_in, const float* scores_in,
                           const uint32_t* keep_in, const int64_t* units, int64_t n_units,
                           double* o_out, double* lse_out, uint8_t* state_out, double* rowmax_out,
                           uint32_t* keep_out) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Sq < 1 || Sk < 1 || D < 1 || Br < 1 || Bc < 1)
        return 1;
    if (causal && Sq != Sk) return 1;
    if (!(lambda >= 0.0) || isinf(lambda)) return 1;
    if (Mg < 1 || N < 1 || N > Mg || sink < 0 || recent < 0) return 1;
    const int nQT = (Sq + Br - 1) / Br, nKT = (Sk + Bc - 1) / Bc, W = (Sk + 31) / 32;
    const int group = Hq / Hkv;
    const double c = scale * M_LOG2E;
    const double L = (lambda == 0.0) ? -INFINITY : log2(lambda);
    const float L32 = (lambda == 0.0) ? -INFINITY : (float)log2((double)(float)lambda);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_units; ++u) {
        const int64_t unit = units ? units[u] : u;
        if (unit < 0 || unit >= (int64_t)B * Hq * nQT) { bad = 1; continue; }
        const int i = (int)(unit % nQT);
        const int hq = (int)((unit / nQT) % Hq);
        const int b = (int)(unit / ((int64_t)nQT * Hq));
        const int hk = hq / group;
        const int r0 = i * Br, r1 = (r0 + Br < Sq) ? r0 + Br : Sq, nr = r1 - r0;

        /* step 1: the N:M keep flags of every row of the query tile */
        unsigned char* keep = calloc((size_t)Br * Sk, 1);
        double* x = malloc(sizeof(double) * Sk);
        for (int rr = 0; rr < Br; ++rr) {
            uint32_t* kw = &keep_out[(u * Br + rr) * W];
            for (int w = 0; w < W; ++w) kw[w] = 0u;
            if (rr >= nr) continue;
            const int r = r0 + rr;
            const int64_t row = (((int64_t)b * Hq + hq) * Sq + r);
            unsigned char* kr = &keep[(size_t)rr * Sk];
            if (mode == 2) {
                for (int kk = 0; kk < Sk; ++kk)
                    kr[kk] = (unsigned char)((keep_in[row * W + (kk >> 5)] >> (kk & 31)) & 1u);
            } else {
                for (int kk = 0; kk < Sk; ++kk) {
                    const int allowed = !causal || kk <= r;
                    if (!allowed) x[kk] = -INFINITY;
                    else if (mode == 1) x[kk] = (double)scores_in[row * Sk + kk];
                    else x[kk] = dot_qk(q, k, Sq, Sk, Hq, Hkv, D, b, r, hq, kk, hk);
                }
                nm_keep_row(r, Sk, causal, N, Mg, sink, recent, x, kr);
            }
            for (int kk = 0; kk < Sk; ++kk)
                if (kr[kk]) kw[kk >> 5] |= 1u << (kk & 31);
        }

        /* step 2: the skip-softmax loop over the masked logits */
        double* m = malloc(sizeof(double) * Br);
        double* l = malloc(sizeof(double) * Br);
        float* m32 = malloc(sizeof(float) * Br);
        double* acc = calloc((size_t)Br * D, sizeof(double));
        double* t = malloc(sizeof(double) * Br * Bc);
        double* M = malloc(sizeof(double) * Br);
        for (int r = 0; r < Br; ++r) { m[r] = -INFINITY; l[r] = 0.0; m32[r] = -INFINITY; }

        for (int j = 0; j < nKT; ++j) {
            const int k0 = j * Bc, k1 = (k0 + Bc < Sk) ? k0 + Bc : Sk;
            uint8_t* st = &state_out[u * nKT + j];
            double* rm = &rowmax_out[(u * nKT + j) * Br];
            for (int r = 0; r < Br; ++r) rm[r] = -INFINITY;
            int visited = causal ? (k0 <= r1 - 1) : 1;
            if (!visited) { *st = 2; continue; }
            for (int rr = 0; rr < nr; ++rr) {
                const int r = r0 + rr;
                M[rr] = -INFINITY;
                for (int kk = k0; kk < k1; ++kk) {
                    double tv = -INFINITY;
                    if (keep[(size_t)rr * Sk + kk])
                        tv = c * dot_qk(q, k, Sq, Sk, Hq, Hkv, D, b, r, hq, kk, hk);
                    t[rr * Bc + (kk - k0)] = tv;
                    if (tv > M[rr]) M[rr] = tv;
                }
                rm[rr] = M[rr];
            }
            int skip;
            if (mode == 2) {
                skip = state_in[unit * nKT + j] == 1;
            } else if (mode == 1) {
                const float* Min = &rowmax_in[(unit * nKT + j) * Br];
                skip = 1;
                for (int rr = 0; rr < nr; ++rr)
                    if (!(Min[rr] < (float)(m32[rr] + L32))) { skip = 0; break; }
            } else {
                skip = 1;
                for (int rr = 0; rr < nr; ++rr)
                    if (!(M[rr] < m[rr] + L)) { skip = 0; break; }
            }
            *st = (uint8_t)skip;
            if (skip) continue;
            for (int rr = 0; rr < nr; ++rr) {
                if (mode == 1) {
                    const float Mf = rowmax_in[(unit * nKT + j) * Br + rr];
                    if (Mf > m32[rr]) m32[rr] = Mf;
                }
                const double m_new = (M[rr] > m[rr]) ? M[rr] : m[rr];
                if (m_new == -INFINITY) continue;
                const double alpha = (m[rr] == -INFINITY) ? 0.0 : exp2(m[rr] - m_new);
                l[rr] *= alpha;
                for (int e = 0; e < D; ++e) acc[rr * D + e] *= alpha;
                for (int kk = k0; kk < k1; ++kk) {
                    const double tv = t[rr * Bc + (kk - k0)];
                    if (tv == -INFINITY) continue;
                    const double p = exp2(tv - m_new);
                    l[rr] += p;
                    for (int e = 0; e < D; ++e)
                        acc[rr * D + e] += p * at(v, Sk, Hkv, D, b, kk, hk, e);
                }
                m[rr] = m_new;
            }
        }
        for (int rr = 0; rr < Br; ++rr) {
            double* o = &o_out[(u * Br + rr) * D];
            if (rr >= nr || l[rr] == 0.0) {
                for (int e = 0; e < D; ++e) o[e] = 0.0;
                lse_out[u * Br + rr] = (rr >= nr) ? 0.0 : -INFINITY;
                continue;
            }
            for (int e = 0; e < D; ++e) o[e] = acc[rr * D + e] / l[rr];
            lse_out[u * Br + rr] = (m[rr] + log2(l[rr])) * M_LN2;
        }
        free(keep); free(x); free(m); free(l); free(m32); free(acc); free(t); free(M);
    }
    return bad;
}

/* ------------------------------------------------------------------------------------------------
 * Route preparation from packed exact-block bitmaps.  [FI-proxy] "Bitmask format".  Integer and
 * exact: for every (b, kv head, q block) row of W = ceil(nKB/32) words, block j < nKB is exact when
 * bit (j & 31) of word (j >> 5) is set (reading: LSB first); bits at j >= nKB are padding and are
 * ignored.  Outputs: n_exact, the exact block indices in ascending order (the rest of the row is
 * filled with -1), and proxy_keep = complement of the exact bits restricted to j < nKB (padding 0).
 * ----------------------------------------------------------------------------------------------*/
int oracle_route_prep(int64_t rows, int nKB, const uint32_t* bitmask, int32_t* n_exact,
                      int32_t* exact_idx, uint32_t* proxy_keep) {
    if (rows < 0 || nKB < 1) return 1;
    const int W = (nKB + 31) / 32;
    for (int64_t row = 0; row < rows; ++row) {
        int count = 0;
        for (int w = 0; w < W; ++w) proxy_keep[row * W + w] = 0u;
        for (int j = 0; j < nKB; ++j) {
            const int bit = (int)((bitmask[row * W + (j >> 5)] >> (j & 31)) & 1u);
            if (bit) exact_idx[row * nKB + count++] = j;
            else proxy_keep[row * W + (j >> 5)] |= 1u << (j & 31);
        }
        for (int j = count; j < nKB; ++j) exact_idx[row * nKB + j] = -1;
        n_exact[row] = count;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Route preparation from canonical BSR (block_indptr / block_indices).  [FI-proxy] "Bitmask format":
 * BSR and bitmap inputs are prepared into the same route stream, and the two give bitwise-identical
 * results.  Integer and exact, written as its definition:
 *
 *   row r (one per (b, kv head, q block), row-major) lists the exact blocks
 *       E_r = { indices[e] : indptr[r] <= e < indptr[r+1], 0 <= indices[e] < nKB }
 *   outputs as for the bitmap: n_exact = |E_r|, E_r ascending then -1, proxy_keep = blocks j < nKB
 *   not in E_r.
 *
 * Readings: a row is a set of block indices, so duplicates collapse and entry order does not
 * matter; entries outside [0, nKB) are dropped; a row whose pointer range is reversed or leaves
 * [0, nnz] is clamped to [0, nnz] (empty when reversed).  *bad_rows counts the rows that are not
 * canonical: a pointer out of range or reversed, an entry outside [0, nnz) or [0, nKB), or entries
 * that are not strictly ascending.
 * ----------------------------------------------------------------------------------------------*/
int oracle_bsr_route_prep(int64_t rows, int nKB, const int32_t* indptr, int64_t nnz,
                          const int32_t* indices, int32_t* n_exact, int32_t* exact_idx,
                          uint32_t* proxy_keep, int64_t* bad_rows) {
    if (rows < 0 || nKB < 1 || nnz < 0) return 1;
    const int W = (nKB + 31) / 32;
    unsigned char* in_set = (unsigned char*)malloc((size_t)nKB);
    if (in_set == NULL) return 2;
    int64_t bad = 0;
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t p0 = indptr[row], p1 = indptr[row + 1];
        int is_bad = p0 < 0 || p1 < p0 || p1 > nnz;
        int64_t start = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
        int64_t end = p1 < start ? start : (p1 > nnz ? nnz : p1);
        memset(in_set, 0, (size_t)nKB);
        for (int64_t e = start; e < end; ++e) {
            const int32_t j = indices[e];
            if (j < 0 || j >= nKB) is_bad = 1;
            else in_set[j] = 1;
            if (e > start && indices[e - 1] >= j) is_bad = 1;
        }
        int count = 0;
        for (int w = 0; w < W; ++w) proxy_keep[row * W + w] = 0u;
        for (int j = 0; j < nKB; ++j) {
            if (in_set[j]) exact_idx[row * nKB + count++] = j;
            else proxy_keep[row * W + (j >> 5)] |= 1u << (j & 31);
        }
        for (int j = count; j < nKB; ++j) exact_idx[row * nKB + j] = -1;
        n_exact[row] = count;
        bad += is_bad;
    }
    free(in_set);
    *bad_rows = bad;
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Proxy-compensated block-sparse forward.  [FI-proxy] "Description" and "Bitmask format".  A
 * closed-form approximation, written as its definition:
 *
 *   c_j   = min(Bk, Sk - j*Bk)                          true token mass of block j
 *   E     = exact blocks of (b, kv head, query block) from the bitmap;
 *   P     = blocks j < nKB not in E  (empty when use_proxy == 0)
 *   s_t   = scale * q.k_t         for every token t of every block in E
 *   s^_j  = scale * q.kmean_j     for every j in P
 *   O     = [sum_t e^s_t v_t + sum_j e^s^_j vsum_j] / [sum_t e^s_t + sum_j c_j e^s^_j]
 *
 * Readings: summaries are caller inputs (bf16 [B,Hkv,nKB,D]); the proxy logit uses the same softmax
 * scale; only the denominator carries c_j (the summed V already carries the mass); non-causal only;
 * a row with nothing to attend to (no exact block and no proxy) gets O = 0, lse = -inf.
 * Units are (b, hq, query block) with query blocks of Bq rows; o_out [n_units][Bq][D].
 * ----------------------------------------------------------------------------------------------*/
int oracle_proxy_fwd(int B, int Hq, int Hkv, int Sq, int Sk, int D, int Bq, int Bk, double scale,
                     const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* k_mean, const uint16_t* v_sum, const uint32_t* bitmask,
                     int use_proxy, const int64_t* units, int64_t n_units, double* o_out,
                     double* lse_out) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Sq < 1 || Sk < 1 || D < 1 || Bq < 1 || Bk < 1)
        return 1;
    const int nQB = (Sq + Bq - 1) / Bq, nKB = (Sk + Bk - 1) / Bk, W = (nKB + 31) / 32;
    const int group = Hq / Hkv;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_units; ++u) {
        const int64_t unit = units ? units[u] : u;
        if (unit < 0 || unit >= (int64_t)B * Hq * nQB) { bad = 1; continue; }
        const int qb = (int)(unit % nQB);
        const int hq = (int)((unit / nQB) % Hq);
        const int b = (int)(unit / ((int64_t)nQB * Hq));
        const int hk = hq / group;
        const uint32_t* bits = &bitmask[(((int64_t)b * Hkv + hk) * nQB + qb) * W];
        double* s = malloc(sizeof(double) * Sk);
        double* sp = malloc(sizeof(double) * nKB);
        double* num = malloc(sizeof(double) * D);
        for (int rr = 0; rr < Bq; ++rr) {
            const int r = qb * Bq + rr;
            double* o = &o_out[(u * Bq + rr) * D];
            if (r >= Sq) {
                for (int e = 0; e < D; ++e) o[e] = 0.0;
                lse_out[u * Bq + rr] = 0.0;
                continue;
            }
            double mu = -INFINITY;
            for (int j = 0; j < nKB; ++j) {
                const int exact = (int)((bits[j >> 5] >> (j & 31)) & 1u);
                const int t0 = j * Bk, t1 = (t0 + Bk < Sk) ? t0 + Bk : Sk;
                sp[j] = -INFINITY;
                if (exact) {
                    for (int t = t0; t < t1; ++t) {
                        s[t] = scale * dot_qk(q, k, Sq, Sk, Hq, Hkv, D, b, r, hq, t, hk);
                        if (s[t] > mu) mu = s[t];
                    }
                } else if (use_proxy) {
                    double d = 0.0;
                    for (int e = 0; e < D; ++e)
                        d += at(q, Sq, Hq, D, b, r, hq, e) *
                             bf16_value(k_mean[(((int64_t)b * Hkv + hk) * nKB + j) * D + e]);
                    sp[j] = scale * d;
                    if (sp[j] > mu) mu = sp[j];
                }
            }
            double den = 0.0;
            for (int e = 0; e < D; ++e) num[e] = 0.0;
            for (int j = 0; j < nKB; ++j) {
                const int exact = (int)((bits[j >> 5] >> (j & 31)) & 1u);
                const int t0 = j * Bk, t1 = (t0 + Bk < Sk) ? t0 + Bk : Sk;
                if (exact) {
                    for (int t = t0; t < t1; ++t) {
                        const double p = exp(s[t] - mu);
                        den += p;
                        for (int e = 0; e < D; ++e) num[e] += p * at(v, Sk, Hkv, D, b, t, hk, e);
                    }
                } else if (use_proxy) {
                    const double p = exp(sp[j] - mu);
                    const double cj = (double)(t1 - t0);
                    den += cj * p;
                    for (int e = 0; e < D; ++e)
                        num[e] += p * bf16_value(v_sum[(((int64_t)b * Hkv + hk) * nKB + j) * D + e]);
                }
            }
            if (den == 0.0) {
                for (int e = 0; e < D; ++e) o[e] = 0.0;
                lse_out[u * Bq + rr] = -INFINITY;
                continue;
            }
            for (int e = 0; e < D; ++e) o[e] = num[e] / den;
            lse_out[u * Bq + rr] = mu + log(den);
        }
        free(s); free(sp); free(num);
    }
    return bad;
}

/* ------------------------------------------------------------------------------------------------
 * Calibrated threshold lowering.  [MO-diff] "Threshold Modes": scale_factor = a*exp(b*s); the
 * backend divides by the key length; the kernel works with log2 of the result.  All in double.
 * ----------------------------------------------------------------------------------------------*/
int oracle_threshold(double a, double b, double target_sparsity, int64_t seq_k,
                     double* scale_factor, double* lambda, double* log2_lambda) {
    if (!(a > 0.0) || !isfinite(b) || !(target_sparsity >= 0.0 && target_sparsity < 1.0) ||
        seq_k < 1)
        return 1;
    *scale_factor = a * exp(b * target_sparsity);
    *lambda = *scale_factor / (double)seq_k;
    *log2_lambda = log2(*lambda);
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Log-space calibration fit.  [MO-diff] introduction ("Calibrated threshold": scale_factor =
 * a*exp(b*target_sparsity) calibrated once, log-space fitting recommended) and "Known Issues"
 * (targets below the smallest sparsity reached extrapolate); [MO-llm] "Custom Configuration"
 * (threshold_trials).  Each trial i ran the kernel at threshold lambda_i and measured tile sparsity
 * s_i; its scale factor is lambda_i * seq_k.  The fit is ordinary least squares of
 *     y_i = ln(lambda_i * seq_k)  on  x_i = s_i:   b = sum (x-xm)(y-ym) / sum (x-xm)^2,
 *                                                 ln a = ym - b*xm,
 * over the usable trials (lambda_i > 0 finite, 0 < s_i < 1; a trial with no skipped tile or with
 * every tile skipped says nothing about where the curve is).  Also returns the smallest and the
 * largest usable sparsity.  Fails (returns 1) with fewer than two usable trials or when all usable
 * sparsities are equal.
 * ----------------------------------------------------------------------------------------------*/
int oracle_fit_threshold(int n, const double* lambdas, const double* sparsities, int64_t seq_k,
                         double* a_out, double* b_out, double* s_min, double* s_max) {
    if (n < 0 || seq_k < 1) return 1;
    int used = 0;
    double xm = 0.0, ym = 0.0, lo = INFINITY, hi = -INFINITY;
    for (int i = 0; i < n; ++i) {
        const double lam = lambdas[i], s = sparsities[i];
        if (!(lam > 0.0) || !isfinite(lam) || !(s > 0.0 && s < 1.0)) continue;
        xm += s;
        ym += log(lam * (double)seq_k);
        lo = s < lo ? s : lo;
        hi = s > hi ? s : hi;
        ++used;
    }
    if (used < 2 || !(hi > lo)) return 1;
    xm /= used;
    ym /= used;
    double sxy = 0.0, sxx = 0.0;
    for (int i = 0; i < n; ++i) {
        const double lam = lambdas[i], s = sparsities[i];
        if (!(lam > 0.0) || !isfinite(lam) || !(s > 0.0 && s < 1.0)) continue;
        sxy += (s - xm) * (log(lam * (double)seq_k) - ym);
        sxx += (s - xm) * (s - xm);
    }
    *b_out = sxy / sxx;
    *a_out = exp(ym - *b_out * xm);
    *s_min = lo;
    *s_max = hi;
    return 0;
}
