/*
 * fp64 CPU oracle for paged single-query decode attention with the V2
 * partition / log-sum-exp split and GQA head mapping.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it. It shares no code, header, table or
 * helper with the HIP library.
 *
 * Sources (the web pages this method is described on):
 *  [TRITON-V2] "paged_attention_v2_triton.py -- Triton PagedAttention V2 for
 *              BI-V100": module docstring (two-phase split), phase-1
 *              partition kernel (gather, scores, online softmax, partition
 *              stores, empty-partition sentinel), phase-2 reduce kernel
 *              (cross-partition log-sum-exp combine).
 *  [METAL-FA]  "Flash Attention Metal Shaders": forward kernel (the same
 *              softmax recurrence in unnormalised form; an empty row gives 0).
 *  [CUDA-A2A]  "all2all_heads.cu": its kernels move tensors of e4m3fn
 *              elements (only the element format is taken from it).
 *
 * What is computed. V2 is an exact reformulation of dense softmax attention
 * over the tokens a sequence's block table gathers, so the plain definition is:
 *   for each sequence s, query head h, kv head kh = h / (H / KH):
 *     K_t, V_t  = the key / value vectors of token t < L gathered through
 *                 block_tables[s][t / BS], slot t % BS
 *     s_t       = scale * sum_d q[s][h][d] * K_t[d]            (scale after the dot)
 *     out[s][h] = sum_t exp(s_t - M) V_t / sum_t exp(s_t - M),  M = max_t s_t
 *     L == 0    -> out = 0
 * Partition mode defines the phase-1 intermediates for p < P on the token
 * range [p*PS, min((p+1)*PS, L)): m_p = max s_t, l_p = sum exp(s_t - m_p),
 * o_p = sum exp(s_t - m_p) V_t / l_p (normalised, as the partition kernel
 * keeps its accumulator divided by the running sum); an empty range gives
 * m_p = -inf, l_p = 0 and o_p left as NaN ("never read").
 * Combine mode is the reduce kernel: over the n = ceil(L/PS) used partitions,
 * M = max m_p, Z = sum exp(m_p - M) l_p, out = sum exp(m_p - M) l_p / Z * o_p.
 *
 * Several query tokens per sequence (speculative decode / chunked prefill
 * over the cache). [TRITON-V2] notes its gather comes from a multi-row
 * (BLOCK_M) prefill kernel; [METAL-FA]'s forward kernel masks keys later than
 * the query position (score -inf). Reading taken: the M query tokens
 * q[s][m] (query layout [S, M, H, D]) are the sequence's last M positions, so
 * token m sits at L - M + m and attends to t <= L - M + m; everything else is
 * unchanged, per query row (outputs [S, M, H, ...]). M = 1 is the decode above.
 *
 * Readings where the pages leave a step open:
 *  - the scale is rounded to fp32 first (the partition kernel types it fp32);
 *  - the 1e-6 clamps on the running sum are inert for finite inputs (the
 *    argmax token contributes exp(0) = 1), so they are omitted;
 *  - the 1024-partition cap of the launcher is an implementation limit of
 *    that GPU, not semantics; any P is accepted.
 * All arithmetic is IEEE double; stored inputs are decoded exactly from
 * their bits using the binary16, bfloat16 and OCP 8-bit E4M3 format
 * definitions.
 *
 * 8-bit KV caches. The launcher of [TRITON-V2] carries a cache dtype string
 * and per-tensor key / value scales (its kernels do not use them), and
 * [CUDA-A2A] "all2all_heads.cu" moves e4m3fn tensors. The plainest reading,
 * taken here: key and value elements are stored as OCP FP8 E4M3 bytes and
 * stand for decode(byte) * k_scale and decode(byte) * v_scale (scales are
 * fp32 scalars, applied in double); the query keeps its own 16-bit dtype and
 * the cache packing factor is x = 16 / 1 = 16. Everything else is unchanged.
 *
 * ALiBi. The Triton PagedAttention V2 page's launcher accepts per-head
 * "alibi_slopes" and never uses them; the pages give no formula. Reading
 * taken: the published ALiBi definition (Press, Smith and Lewis, "Train
 * Short, Test Long: Attention with Linear Biases", ICLR 2022): a query at
 * position i adds slope_h * (j - i) to its score for the key at position j
 * (0 at its own position, more negative further back), after the scaling of
 * the dot product; the slopes are the caller's fp32 [H] values. The query
 * position is L - 1 for single-query decode and L - M + m for query token m
 * of M.
 *
 * Log-sum-exp output and merge. [METAL-FA]'s forward kernel stores, per query
 * row, the log-sum-exp of its scores, m + log(l) (its clamp of l is inert once
 * a row has a key). Reading taken: lse = log(sum_t exp(s_t)) over the scores
 * defined above, -inf for a row with no keys. Two results of the same rows
 * over disjoint key sets merge by the [TRITON-V2] reduce's combine, each
 * side's (m, l) folded into its lse (oracle_merge_states).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_FP8_E4M3 = 3 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal (fraction * 2^-24), 31 -> inf / NaN. */
double oracle_decode_binary16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int f = bits & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * exponent 0 -> subnormal (fraction * 2^-133), 255 -> inf / NaN. */
double oracle_decode_bfloat16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xff;
    int f = bits & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);
    }
    return sign ? -v : v;
}

/* OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits
 * (bias 7), 3 fraction bits; exponent 0 -> subnormal (fraction * 2^-9); no
 * infinities: only S.1111.111 is NaN, so exponent 15 with fraction < 7 is a
 * normal number (largest 1.75 * 2^8 = 448). */
double oracle_decode_e4m3(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xf;
    int f = bits & 0x7;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -9);
    } else if (e == 15 && f == 7) {
        v = NAN;
    } else {
        v = ldexp((double)(8 + f), e - 10);
    }
    return sign ? -v : v;
}

static double load_elem(const void* base, int64_t idx, int dtype) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    if (dtype == ORACLE_FP8_E4M3) return oracle_decode_e4m3(((const uint8_t*)base)[idx]);
    uint16_t b = ((const uint16_t*)base)[idx];
    return dtype == ORACLE_F16 ? oracle_decode_binary16(b) : oracle_decode_bfloat16(b);
}

void oracle_decode_array(double* out, const void* src, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = load_elem(src, i, dtype);
}

static int elem_size(int dtype) {
    return dtype == ORACLE_F32 ? 4 : dtype == ORACLE_FP8_E4M3 ? 1 : 2;
}

/* Problem description shared by the entry points. */
typedef struct {
    const void* q;      /* [S, H, D]               */
    const void* kc;     /* [B, KH, D/x, BS, x]     */
    const void* vc;     /* [B, KH, D, BS]          */
    const int32_t* bt;  /* [S, MB]                 */
    const int32_t* sl;  /* [S]                     */
    int32_t S, H, KH, D, BS, MB, P, PS;
    int32_t qdtype, kvdtype;  /* query dtype; key / value cache dtype */
    int32_t M;                /* query tokens per sequence (1: single-query decode) */
    double scale;
    double kscale, vscale;    /* cache dequantisation scales (1 for 16/32-bit caches) */
    const float* alibi;       /* [H] ALiBi slopes, or NULL (no position bias) */
    /* outputs (any may be NULL) */
    double* out;        /* [S, H, D]     dense attention      */
    double* tmp;        /* [S, H, P, D]  partition outputs    */
    double* es;         /* [S, H, P]     partition exp sums   */
    double* ml;         /* [S, H, P]     partition max logits */
    double* lse;        /* [S, H]        log-sum-exp of the scores (with out) */
    /* work list */
    const int32_t* seqs;
    int32_t n_seqs;
    int64_t next;       /* atomic work counter over n_seqs * KH */
} problem_t;

/* Token t of sequence s: physical block and slot (the paged gather). */
static void gather_index(const problem_t* pr, int32_t s, int32_t t, int32_t* blk, int32_t* slot) {
    *blk = pr->bt[(int64_t)s * pr->MB + t / pr->BS];
    *slot = t % pr->BS;
}

/* K element d of (block b, kv head kh, slot o): key_cache[b][kh][d / x][o][d % x]. */
static double key_at(const problem_t* pr, int32_t b, int32_t kh, int32_t o, int32_t d) {
    int32_t x = 16 / elem_size(pr->kvdtype);
    int64_t idx = ((((int64_t)b * pr->KH + kh) * (pr->D / x) + d / x) * pr->BS + o) * x + d % x;
    return load_elem(pr->kc, idx, pr->kvdtype) * pr->kscale;
}

/* V element d of (block b, kv head kh, slot o): value_cache[b][kh][d][o]. */
static double value_at(const problem_t* pr, int32_t b, int32_t kh, int32_t o, int32_t d) {
    int64_t idx = (((int64_t)b * pr->KH + kh) * pr->D + d) * pr->BS + o;
    return load_elem(pr->vc, idx, pr->kvdtype) * pr->vscale;
}

/* Query row r = s * M + m (query token m of sequence s), head h. */
static double query_at(const problem_t* pr, int64_t r, int32_t h, int32_t d) {
    return load_elem(pr->q, (r * pr->H + h) * pr->D + d, pr->qdtype);
}

/* Softmax-weighted value mix of tokens [t0, t1) given their scores.
 * Writes m = max score, l = sum exp(score - m), o[d] = sum exp(score - m) V[d] / l. */
static void softmax_mix(const problem_t* pr, int32_t s, int32_t kh, const double* score,
                        int32_t t0, int32_t t1, double* m_out, double* l_out, double* o) {
    double m = -INFINITY;
    for (int32_t t = t0; t < t1; ++t)
        if (score[t] > m) m = score[t];
    double l = 0.0;
    for (int32_t d = 0; d < pr->D; ++d) o[d] = 0.0;
    for (int32_t t = t0; t < t1; ++t) {
        double w = exp(score[t] - m);
        l += w;
        int32_t b, slot;
        gather_index(pr, s, t, &b, &slot);
        for (int32_t d = 0; d < pr->D; ++d) o[d] += w * value_at(pr, b, kh, slot, d);
    }
    for (int32_t d = 0; d < pr->D; ++d) o[d] /= l;
    *m_out = m;
    *l_out = l;
}

/* Keys query token m of a length-L sequence attends to: the M query tokens
 * are the sequence's last M positions, token m sits at L - M + m and sees
 * positions t <= L - M + m (the causal rule); clamped to [0, L]. M = 1 gives L. */
static int32_t causal_len(int32_t L, int32_t M, int32_t m) {
    int32_t e = L - M + m + 1;
    return e < 0 ? 0 : (e > L ? L : e);
}

static void run_item(problem_t* pr, int32_t s, int32_t kh) {
    int32_t L0 = pr->sl[s];
    int32_t G = pr->H / pr->KH;
    double* score = (double*)malloc(sizeof(double) * (size_t)(L0 > 0 ? L0 : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)pr->D);
    for (int32_t mq = 0; mq < pr->M; ++mq) {
      int64_t r = (int64_t)s * pr->M + mq;   /* query row */
      int32_t L = causal_len(L0, pr->M, mq); /* keys this query token sees */
      for (int32_t g = 0; g < G; ++g) {
        int32_t h = kh * G + g; /* consecutive query heads share one kv head */
        for (int32_t t = 0; t < L; ++t) {
            int32_t b, slot;
            gather_index(pr, s, t, &b, &slot);
            double dot = 0.0;
            for (int32_t d = 0; d < pr->D; ++d)
                dot += query_at(pr, r, h, d) * key_at(pr, b, kh, slot, d);
            score[t] = pr->scale * dot;
            if (pr->alibi) /* the query sits at position L0 - M + mq */
                score[t] += (double)pr->alibi[h] * (double)(t - (L0 - pr->M + mq));
        }
        if (pr->out) {
            double* dst = pr->out + (r * pr->H + h) * pr->D;
            if (L == 0) {
                for (int32_t d = 0; d < pr->D; ++d) dst[d] = 0.0;
                if (pr->lse) pr->lse[r * pr->H + h] = -INFINITY;
            } else {
                double m, l;
                softmax_mix(pr, s, kh, score, 0, L, &m, &l, dst);
                if (pr->lse) pr->lse[r * pr->H + h] = m + log(l);
            }
        }
        if (pr->tmp || pr->es || pr->ml) {
            for (int32_t p = 0; p < pr->P; ++p) {
                int64_t sp = (r * pr->H + h) * pr->P + p;
                int32_t t0 = p * pr->PS;
                int32_t t1 = t0 + pr->PS < L ? t0 + pr->PS : L;
                double m = -INFINITY, l = 0.0;
                if (t0 < L) {
                    softmax_mix(pr, s, kh, score, t0, t1, &m, &l, o);
                } else {
                    for (int32_t d = 0; d < pr->D; ++d) o[d] = NAN;
                }
                if (pr->ml) pr->ml[sp] = m;
                if (pr->es) pr->es[sp] = l;
                if (pr->tmp) memcpy(pr->tmp + sp * pr->D, o, sizeof(double) * (size_t)pr->D);
            }
        }
      }
    }
    free(o);
    free(score);
}

static void* worker(void* arg) {
    problem_t* pr = (problem_t*)arg;
    int64_t total = (int64_t)pr->n_seqs * pr->KH;
    for (;;) {
        int64_t i = __atomic_fetch_add(&pr->next, 1, __ATOMIC_RELAXED);
        if (i >= total) break;
        int32_t s = pr->seqs[i / pr->KH];
        run_item(pr, s, (int32_t)(i % pr->KH));
    }
    return NULL;
}

static void run_all(problem_t* pr, const int32_t* seqs, int32_t n_seqs, int nthreads) {
    int32_t* all = NULL;
    if (!seqs) {
        all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(pr->S > 0 ? pr->S : 1));
        for (int32_t s = 0; s < pr->S; ++s) all[s] = s;
        seqs = all;
        n_seqs = pr->S;
    }
    pr->seqs = seqs;
    pr->n_seqs = n_seqs;
    pr->next = 0;
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, pr);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(all);
}

static int valid_dtypes(int32_t qdtype, int32_t kvdtype) {
    if (qdtype < ORACLE_F32 || qdtype > ORACLE_BF16) return 0;
    if (kvdtype == ORACLE_FP8_E4M3) return qdtype != ORACLE_F32;
    return kvdtype == qdtype;
}

/* Dense attention over the gathered tokens, the most general form: query
 * [S, M, H, D] rows (M = 1: single-query decode), caches decoded as kvdtype
 * and scaled by k_scale / v_scale, optional ALiBi slopes [H] (NULL: none).
 * out [S, M, H, D] and lse [S, M, H] (either may be NULL): only rows of the
 * listed sequences are written (seqs == NULL means all). lse is the
 * log-sum-exp of each row's scores, m + log(l) = log(sum_t exp(s_t)), -inf
 * for a row with no keys (the Flash Attention Metal forward kernel stores the
 * same quantity per row; its clamp of l is inert when there is at least one
 * key, since l >= 1 then). Returns 0, or -1 on a shape or dtype pair the
 * definition does not cover. */
int oracle_attention_full(double* out, double* lse, const void* q, const void* kc,
                          const void* vc, const int32_t* block_tables, const int32_t* seq_lens,
                          int32_t S, int32_t M, int32_t H, int32_t KH, int32_t D, int32_t BS,
                          int32_t MB, float scale, int32_t qdtype, int32_t kvdtype,
                          float k_scale, float v_scale, const float* alibi_slopes,
                          const int32_t* seqs, int32_t n_seqs, int32_t nthreads) {
    if (!valid_dtypes(qdtype, kvdtype) || M < 1) return -1;
    if (KH <= 0 || H % KH || D % (16 / elem_size(kvdtype))) return -1;
    problem_t pr;
    memset(&pr, 0, sizeof pr);
    pr.q = q; pr.kc = kc; pr.vc = vc; pr.bt = block_tables; pr.sl = seq_lens;
    pr.S = S; pr.H = H; pr.KH = KH; pr.D = D; pr.BS = BS; pr.MB = MB;
    pr.qdtype = qdtype; pr.kvdtype = kvdtype; pr.M = M;
    pr.scale = (double)scale;
    pr.kscale = (double)k_scale; pr.vscale = (double)v_scale;
    pr.alibi = alibi_slopes;
    pr.out = out; pr.lse = lse;
    run_all(&pr, seqs, n_seqs, nthreads);
    return 0;
}

/* oracle_attention_full without lse or ALiBi. */
int oracle_attention_ex(double* out, const void* q, const void* kc, const void* vc,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t S, int32_t M, int32_t H, int32_t KH, int32_t D, int32_t BS,
                        int32_t MB, float scale, int32_t qdtype, int32_t kvdtype, float k_scale,
                        float v_scale, const int32_t* seqs, int32_t n_seqs, int32_t nthreads) {
    return oracle_attention_full(out, NULL, q, kc, vc, block_tables, seq_lens, S, M, H, KH, D,
                                 BS, MB, scale, qdtype, kvdtype, k_scale, v_scale, NULL, seqs,
                                 n_seqs, nthreads);
}

/* oracle_attention_full without ALiBi. */
int oracle_attention_lse(double* out, double* lse, const void* q, const void* kc,
                         const void* vc, const int32_t* block_tables, const int32_t* seq_lens,
                         int32_t S, int32_t M, int32_t H, int32_t KH, int32_t D, int32_t BS,
                         int32_t MB, float scale, int32_t qdtype, int32_t kvdtype,
                         float k_scale, float v_scale, const int32_t* seqs, int32_t n_seqs,
                         int32_t nthreads) {
    return oracle_attention_full(out, lse, q, kc, vc, block_tables, seq_lens, S, M, H, KH, D,
                                 BS, MB, scale, qdtype, kvdtype, k_scale, v_scale, NULL, seqs,
                                 n_seqs, nthreads);
}

/* Merge two attention results of the same query rows over disjoint key sets
 * (rows x D values and their log-sum-exps): with Mx = max(lse_a, lse_b),
 * w = exp(lse - Mx), out = (w_a a + w_b b) / (w_a + w_b) and
 * out_lse = Mx + log(w_a + w_b); both -inf (no keys on either side) gives
 * out = 0, out_lse = -inf. This is the reduce's log-sum-exp combine for two
 * "partitions" whose weights are already folded into their lse. */
void oracle_merge_states(double* out, double* out_lse, const double* a, const double* lse_a,
                         const double* b, const double* lse_b, int64_t rows, int32_t D) {
    for (int64_t r = 0; r < rows; ++r) {
        double mx = lse_a[r] > lse_b[r] ? lse_a[r] : lse_b[r];
        if (mx == -INFINITY) {
            for (int32_t d = 0; d < D; ++d) out[r * D + d] = 0.0;
            out_lse[r] = -INFINITY;
            continue;
        }
        double wa = exp(lse_a[r] - mx), wb = exp(lse_b[r] - mx);
        for (int32_t d = 0; d < D; ++d)
            out[r * D + d] = (wa * a[r * D + d] + wb * b[r * D + d]) / (wa + wb);
        out_lse[r] = mx + log(wa + wb);
    }
}

/* Same, one dtype for query and caches, no cache scales. */
int oracle_attention(double* out, const void* q, const void* kc, const void* vc,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     int32_t S, int32_t H, int32_t KH, int32_t D, int32_t BS, int32_t MB,
                     float scale, int32_t dtype, const int32_t* seqs, int32_t n_seqs,
                     int32_t nthreads) {
    return oracle_attention_ex(out, q, kc, vc, block_tables, seq_lens, S, 1, H, KH, D, BS, MB,
                               scale, dtype, dtype, 1.0f, 1.0f, seqs, n_seqs, nthreads);
}

/* Phase-1 intermediates: tmp[S,M,H,P,D], es[S,M,H,P], ml[S,M,H,P] for the
 * listed sequences (ALiBi slopes [H] or NULL). Returns -1 if a length
 * exceeds P*PS. */
int oracle_partition_stats_full(double* tmp, double* es, double* ml, const void* q,
                                const void* kc, const void* vc, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t S, int32_t M, int32_t H,
                                int32_t KH, int32_t D, int32_t BS, int32_t MB, int32_t P,
                                int32_t PS, float scale, int32_t qdtype, int32_t kvdtype,
                                float k_scale, float v_scale, const float* alibi_slopes,
                                const int32_t* seqs, int32_t n_seqs, int32_t nthreads) {
    if (!valid_dtypes(qdtype, kvdtype) || M < 1) return -1;
    if (KH <= 0 || H % KH || D % (16 / elem_size(kvdtype)) || PS <= 0 || P < 1) return -1;
    for (int32_t s = 0; s < S; ++s)
        if (seq_lens[s] > (int64_t)P * PS) return -1;
    problem_t pr;
    memset(&pr, 0, sizeof pr);
    pr.q = q; pr.kc = kc; pr.vc = vc; pr.bt = block_tables; pr.sl = seq_lens;
    pr.S = S; pr.H = H; pr.KH = KH; pr.D = D; pr.BS = BS; pr.MB = MB;
    pr.qdtype = qdtype; pr.kvdtype = kvdtype; pr.M = M;
    pr.P = P; pr.PS = PS;
    pr.scale = (double)scale;
    pr.kscale = (double)k_scale; pr.vscale = (double)v_scale;
    pr.alibi = alibi_slopes;
    pr.tmp = tmp; pr.es = es; pr.ml = ml;
    run_all(&pr, seqs, n_seqs, nthreads);
    return 0;
}

/* oracle_partition_stats_full without ALiBi. */
int oracle_partition_stats_ex(double* tmp, double* es, double* ml, const void* q,
                              const void* kc, const void* vc, const int32_t* block_tables,
                              const int32_t* seq_lens, int32_t S, int32_t M, int32_t H,
                              int32_t KH, int32_t D, int32_t BS, int32_t MB, int32_t P,
                              int32_t PS, float scale, int32_t qdtype, int32_t kvdtype,
                              float k_scale, float v_scale, const int32_t* seqs, int32_t n_seqs,
                              int32_t nthreads) {
    return oracle_partition_stats_full(tmp, es, ml, q, kc, vc, block_tables, seq_lens, S, M, H,
                                       KH, D, BS, MB, P, PS, scale, qdtype, kvdtype, k_scale,
                                       v_scale, NULL, seqs, n_seqs, nthreads);
}

int oracle_partition_stats(double* tmp, double* es, double* ml, const void* q, const void* kc,
                           const void* vc, const int32_t* block_tables, const int32_t* seq_lens,
                           int32_t S, int32_t H, int32_t KH, int32_t D, int32_t BS, int32_t MB,
                           int32_t P, int32_t PS, float scale, int32_t dtype,
                           const int32_t* seqs, int32_t n_seqs, int32_t nthreads) {
    return oracle_partition_stats_ex(tmp, es, ml, q, kc, vc, block_tables, seq_lens, S, 1, H,
                                     KH, D, BS, MB, P, PS, scale, dtype, dtype, 1.0f, 1.0f, seqs,
                                     n_seqs, nthreads);
}

/* Phase-2 cross-partition log-sum-exp combine, per query row (s, m) and head
 * h, over the n = ceil(len / PS) partitions its len = causal_len(L, M, m) keys
 * use; n == 0 gives 0. Rows are [S * M, H]; M = 1 is the single-query decode. */
void oracle_combine_ex(double* out, const double* tmp, const double* es, const double* ml,
                       const int32_t* seq_lens, int32_t S, int32_t M, int32_t H, int32_t D,
                       int32_t P, int32_t PS) {
    for (int32_t s = 0; s < S; ++s) {
      for (int32_t mq = 0; mq < M; ++mq) {
        int64_t r = (int64_t)s * M + mq;
        int32_t n = (causal_len(seq_lens[s], M, mq) + PS - 1) / PS;
        for (int32_t h = 0; h < H; ++h) {
            double* dst = out + (r * H + h) * D;
            int64_t base = (r * H + h) * P;
            for (int32_t d = 0; d < D; ++d) dst[d] = 0.0;
            if (n == 0) continue;
            double Mx = -INFINITY;
            for (int32_t p = 0; p < n; ++p)
                if (ml[base + p] > Mx) Mx = ml[base + p];
            double Z = 0.0;
            for (int32_t p = 0; p < n; ++p) Z += exp(ml[base + p] - Mx) * es[base + p];
            for (int32_t p = 0; p < n; ++p) {
                double w = exp(ml[base + p] - Mx) * es[base + p] / Z;
                for (int32_t d = 0; d < D; ++d) dst[d] += w * tmp[(base + p) * D + d];
            }
        }
      }
    }
}

void oracle_combine(double* out, const double* tmp, const double* es, const double* ml,
                    const int32_t* seq_lens, int32_t S, int32_t H, int32_t D, int32_t P,
                    int32_t PS) {
    oracle_combine_ex(out, tmp, es, ml, seq_lens, S, 1, H, D, P, PS);
}

/* The gather itself: for every (s, t < L_s) in order, the physical block and
 * slot the token is read from. Returns the number of entries written. */
int64_t oracle_gather_indices(int32_t* blk, int32_t* slot, const int32_t* block_tables,
                              const int32_t* seq_lens, int32_t S, int32_t MB, int32_t BS) {
    problem_t pr;
    memset(&pr, 0, sizeof pr);
    pr.bt = block_tables; pr.sl = seq_lens; pr.S = S; pr.MB = MB; pr.BS = BS;
    int64_t n = 0;
    for (int32_t s = 0; s < S; ++s)
        for (int32_t t = 0; t < seq_lens[s]; ++t, ++n) gather_index(&pr, s, t, &blk[n], &slot[n]);
    return n;
}
