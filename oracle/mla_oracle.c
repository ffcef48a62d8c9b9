/*
 * mla_oracle.c -- plain FP64 CPU oracle of MLA decode attention over an FP8 E4M3 latent cache.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke entry point and the benchmark's CPU-baseline leg
 * load this library. It shares no code, header, table or helper with the HIP library; it is slow on
 * purpose and written to be checked against the pages by eye.
 *
 * Sources (vLLM API documentation pages; cited by page title and section):
 *   [SPARSE]  vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.attn_sparse
 *             - module docstring: 576-byte cache rows (512 latent bytes = V, then 64 rope bytes);
 *               the per-chunk online softmax in base 2 with the running maximum; P anchored at 448
 *               times the exponential of the logit minus the running maximum, rounded to E4M3
 *               (round to nearest, saturating); FP32 sums of the P before rounding; the merge that
 *               weights each split by exp2(its max - the top max), divides by the total and scales by
 *               k_scale, with LSE = max + log2(total / 448) reported in natural log.
 *             - module docstring, last paragraph: rows with no key write zeros and LSE = -inf.
 *             - SparseDcpDecode.kernel: a row's count is clamped to [0, width]; split s of SPLIT takes
 *               keys [s*per, min(n, (s+1)*per)) with per = ceil(n / SPLIT), in chunks of CHUNK keys.
 *             - SparseDcpDecode.merge: the fixed-order FP32 combine of the splits. Its identity
 *               (weights exp2(m_s - top)) holds for any division of the keys into consecutive
 *               splits, so a plan may also be given as explicit split boundaries per key group.
 *             - module docstring, "push" and SparseDcpDecode: with decode-context parallelism each
 *               rank decodes its share of a row's keys and sends the merged row (o, LSE) to the
 *               head's owner, which merges the ranks' rows (mo_combine below).
 *   [AMD]     vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_attn
 *             - module docstring: position i of a request's qlen query rows sees keys up to
 *               seq_len - qlen + i; a split with no visible key leaves LSE = -inf and o = 0.
 *             - fp8_unpack4: E4M3 to f32 is exact.
 *             - module docstring and fp8_split4: P (scaled by a power of two) goes to the PV
 *               product as two E4M3 values, hi and lo, with P ~ hi + lo; V meets both. With the
 *               MO_PSPLIT flag the METHOD mode takes this form of P (mo_p_split below).
 *
 * The query: the bf16 row as given (q exact in FP64), or, with the MO_QE4M3 flag added to a mode,
 * its E4M3 form (see mo_q_e4m3 below).
 *
 * Three modes of the same computation for one query row (b, i, h):
 *   MO_EXACT      the textbook definition: LSE = ln sum_j exp(x_j), o = sum_j softmax(x)_j V_j, with
 *                 x_j = scale * q . K_j, K_j = k_scale * dec(K bytes), V_j = k_scale * dec(V bytes).
 *   MO_ONLINE     the pages' split / chunked online softmax and merge, P not rounded (equals MO_EXACT
 *                 up to FP64 rounding for every split plan: the split-merge identity).
 *   MO_METHOD     MO_ONLINE with each P rounded to E4M3 before it multiplies V (with MO_PSPLIT: split
 *                 into E4M3 hi + lo, see mo_p_used). The rounding decision is taken on P rounded to
 *                 FP32, the precision the pages compute P in.
 *                 Optionally also a per-element allowance: an implementation that forms the logits
 *                 from FP8 MFMA products and P in FP32 knows each P only to within a relative error
 *                 bounded per key (logit_error_bound below), and where a P lies that close to an
 *                 E4M3 rounding midpoint either rounding is a correct result. The allowance is what
 *                 such keys can move o by: the E4M3 step between the two roundings times |V|,
 *                 carried through the same rescaling and merge as O.
 *
 * Readings of the pages this oracle takes (each also listed in the design notes):
 *   - the causal bound is inclusive: row i sees n_i = seq_len - qlen + i + 1 keys (clamped to
 *     [0, seq_len]);
 *   - dense splits divide the request's seq_len keys (the KV a split streams); a row masks the keys
 *     past its own causal bound inside them;
 *   - a key whose cache row falls outside [0, num_rows) (an index outside the cache, a page outside
 *     the pool) is absent: it contributes nothing and is never read;
 *   - one per-tensor k_scale dequantizes K (all 576 bytes) and V;
 *   - the softmax scale multiplies q . K; the LSE excludes the 448 anchor.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MO_ROW 576    /* bytes of a cache row */
#define MO_LATENT 512 /* latent bytes = V width */

enum { MO_EXACT = 0, MO_ONLINE = 1, MO_METHOD = 2 };
enum { MO_QE4M3 = 16 }; /* flag added to a mode: the logits use the E4M3 query */
enum { MO_PSPLIT = 32 }; /* flag added to MO_METHOD: P enters PV as E4M3 hi + lo */

/* ---- number formats --------------------------------------------------------------------------- */

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is subnormal (m * 2^-9);
 * 0x7F / 0xFF are NaN; no infinity. */
double mo_e4m3_decode(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round to the nearest E4M3 value, ties to an even mantissa; magnitudes of 448 and above saturate to
 * 448 (the "satfinite" conversion); NaN maps to 0x7F. */
uint8_t mo_e4m3_encode(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7F;
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9 */
        double t = a * 512.0;
        double r = nearbyint(t); /* default rounding mode: to nearest, ties to even */
        int m = (int)r;          /* 0..8; 8 is the smallest normal, code 0x08 */
        return sign | (uint8_t)m;
    }
    int e;
    double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int exp_unbiased = e - 1; /* a = (2f) * 2^(e-1), 2f in [1, 2) */
    double t = (2.0 * f - 1.0) * 8.0; /* mantissa in units of 1/8, in [0, 8) */
    int m = (int)nearbyint(t);
    if (m == 8) {
        m = 0;
        exp_unbiased += 1;
    }
    int be = exp_unbiased + 7;
    if (be > 15 || (be == 15 && m == 7))
        return sign | 0x7E; /* only reachable by rounding up to 480: saturate */
    return sign | (uint8_t)((be << 3) | m);
}

/* bfloat16 bits -> value (exact) */
double mo_bf16_decode(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* ---- the E4M3 query ---------------------------------------------------------------------------- */

/*
 * [SPARSE] module docstring, Precision paragraph: FlashInfer's sparse MLA decode takes an E4M3
 * query. How the bf16 query becomes E4M3 is not stated; the reading taken here uses the per-row
 * power of two of [AMD] (its query split scales q by 2^k): k is the largest integer with
 * max_c |q_c| * 2^k <= 448, at most 126, and 0 for an all-zero row. Each value is rounded to E4M3
 * (nearest, ties to even) at that scale and scaled back: qe_c = dec(E4M3(q_c * 2^k)) * 2^-k.
 * Scaling by powers of two is exact in FP64 here, so the only rounding is the E4M3 one.
 */
int mo_q_shift(const double* qd)
{
    double amax = 0.0;
    for (int c = 0; c < MO_ROW; c++)
        if (fabs(qd[c]) > amax)
            amax = fabs(qd[c]);
    if (amax == 0.0)
        return 0;
    int k = 0;
    while (k < 126 && ldexp(amax, k + 1) <= 448.0)
        k++;
    while (ldexp(amax, k) > 448.0)
        k--;
    return k;
}

void mo_q_e4m3(const double* qd, double* qe)
{
    const int k = mo_q_shift(qd);
    for (int c = 0; c < MO_ROW; c++)
        qe[c] = ldexp(mo_e4m3_decode(mo_e4m3_encode(ldexp(qd[c], k))), -k);
}

/* bf16 bits of one row -> its E4M3 query (for the tests) */
void mo_q_e4m3_bits(const uint16_t* q, double* qe)
{
    double qd[MO_ROW];
    for (int c = 0; c < MO_ROW; c++)
        qd[c] = mo_bf16_decode(q[c]);
    mo_q_e4m3(qd, qe);
}

/* ---- one query row ---------------------------------------------------------------------------- */

/* The P that meets V in METHOD mode, from P rounded to FP32 (the pages compute P in FP32):
 *   plain: E4M3(P);
 *   split: hi + lo with hi = E4M3(P), lo = E4M3(P - hi) (P - hi is exact: both are FP32 values
 *          within a factor of two of each other, or hi = 0).
 * Either way a monotone non-decreasing function of P: within one hi value lo follows P, and where
 * hi steps up by u at a midpoint, lo steps down from +u/2 to -u/2 (both E4M3 values), so the sum
 * does not move there. */
double mo_p_used(double p, int split)
{
    const double pf = (double)(float)p;
    const double hi = mo_e4m3_decode(mo_e4m3_encode(pf));
    if (!split)
        return hi;
    return hi + mo_e4m3_decode(mo_e4m3_encode(pf - hi));
}

/*
 * How far an implementation's P may lie from the exact one, per key: the bound the allowance uses.
 * It models the kernels' arithmetic (an FP8 MFMA implementation of the AMD page's logits, P in
 * FP32 as the sparse page computes it):
 *   - the query enters as its exact E4M3 split y = q 2^k = hi + lo + r (k as in mo_q_shift; r = 0
 *     wherever |y| >= 2^-2, and |r| <= 2^-10 below), or as hi alone with the E4M3 query;
 *   - the products hi_c K_c and lo_c K_c (exact: 4-bit by 4-bit significands) are summed by
 *     16x16x128 FP8 MFMAs whose accumulation was measured on MI355X (an in-register probe of single
 *     instructions): the 128 products of one instruction form 16 groups of 8 consecutive k
 *     positions -- 8 consecutive columns of one operand (hi or lo), as any layout that keeps
 *     8-byte runs of a row together gives; inside a group each product is cut toward zero to a
 *     multiple of 2^(e - 13), e = floor(log2) of the group's largest |product| (which itself stays
 *     exact), and the group sums and the accumulator are added with FP32 round-to-nearest-even;
 *     so a logit's sum S is off by at most
 *         T + gamma(n) sum |p|,  T = sum over groups of (sum_c min(|p_c|, w) - w), w = 2^(e - 13),
 *     gamma(n) = n u / (1 - n u), u = 2^-24, n = 16 additions per instruction times the
 *     instructions in the chain (9 with the split query: 4 latent steps of hi and of lo and a rope
 *     step holding both; 5 with the E4M3 query), plus sum_c |r_c K_c| for the query split's loss;
 *   - the logit x = S times the row scale (scale k_scale log2(e) 2^-k, rounded to FP32 once) with
 *     the running maximum m subtracted in one fused operation: at most 2^-23 (|x| + |x - m|) more;
 *   - m is the largest such x of the part so far, off by at most the largest bound among them;
 *   - P = 448 exp2(x - m): exp2 to 1 ulp (the ISA's stated accuracy of V_EXP_F32) and one
 *     rounding of the product by 448: 2^-22 relative covers both.
 * In log2 units d(x) = rs (T + gamma(n) sum|p| + sum|r K|) + 2^-23 (|x| + |x - m|), with rs =
 * scale k_scale log2(e) 2^-k; the relative bound of P is exp2(d(x) + d(m)) - 1 + 2^-22.
 */
static double group_cut_bound(const double* p, int n)
{
    /* T of the comment above over n products (n a multiple of 8) */
    double t = 0.0;
    for (int g = 0; g < n; g += 8) {
        double m = 0.0;
        for (int c = g; c < g + 8; c++)
            if (fabs(p[c]) > m)
                m = fabs(p[c]);
        if (m == 0.0)
            continue;
        int e;
        frexp(m, &e); /* m = f 2^e, f in [0.5, 1): floor(log2 m) = e - 1 */
        const double w = ldexp(1.0, e - 1 - 13);
        double sg = 0.0;
        for (int c = g; c < g + 8; c++)
            sg += fabs(p[c]) < w ? fabs(p[c]) : w;
        t += sg - w;
    }
    return t;
}

typedef struct {
    double hi[MO_ROW], lo[MO_ROW], res[MO_ROW]; /* the query split (q 2^k units) */
    double rs;                                  /* log2 units per product unit */
    int steps;                                  /* MFMA instructions in a logit's chain */
} mo_qsplit;

static void split_query(const uint16_t* q, int qe4m3, double scale, double k_scale, mo_qsplit* s)
{
    double qd[MO_ROW];
    for (int c = 0; c < MO_ROW; c++)
        qd[c] = mo_bf16_decode(q[c]);
    const int k = mo_q_shift(qd);
    for (int c = 0; c < MO_ROW; c++) {
        const double y = ldexp(qd[c], k);
        s->hi[c] = mo_e4m3_decode(mo_e4m3_encode(y));
        s->lo[c] = qe4m3 ? 0.0 : mo_e4m3_decode(mo_e4m3_encode(y - s->hi[c]));
        s->res[c] = qe4m3 ? 0.0 : fabs(y - s->hi[c] - s->lo[c]);
    }
    s->rs = scale * k_scale / log(2.0) * ldexp(1.0, -k);
    s->steps = qe4m3 ? 5 : 9;
}

/* rs (T + gamma(n) sum|p| + sum|r K|) of one key: the sum's part of d(x) */
static double logit_error_bound(const mo_qsplit* s, const uint8_t* krow)
{
    double ph[MO_ROW], pl[MO_ROW], sum = 0.0, rk = 0.0;
    for (int c = 0; c < MO_ROW; c++) {
        const double kc = mo_e4m3_decode(krow[c]);
        ph[c] = s->hi[c] * kc;
        pl[c] = s->lo[c] * kc;
        sum += fabs(ph[c]) + fabs(pl[c]);
        rk += s->res[c] * fabs(kc);
    }
    const double u = ldexp(1.0, -24), n = 16.0 * s->steps;
    const double gamma = n * u / (1.0 - n * u);
    return s->rs * (group_cut_bound(ph, MO_ROW) + group_cut_bound(pl, MO_ROW) + gamma * sum + rk);
}

/* The sum's part of d(x) for query row q (bf16 bits) and cache row krow (for the tests). */
double mo_logit_bound(const uint16_t* q, const uint8_t* krow, int qe4m3, double scale,
                      double k_scale)
{
    mo_qsplit s;
    split_query(q, qe4m3, scale, k_scale, &s);
    return logit_error_bound(&s, krow);
}

/* The largest change of the P used (mo_p_used) when P moves by up to rel relative: 0 unless a
 * rounding midpoint lies within that distance. mo_p_used is monotone, so the ends of the interval
 * bound every point inside it. */
static double rounding_ambiguity(double p, int split, double rel)
{
    const double c0 = mo_p_used(p, split);
    const double lo = mo_p_used(p * (1.0 - rel), split);
    const double hi = mo_p_used(p * (1.0 + rel), split);
    const double a = fabs(lo - c0), b = fabs(hi - c0);
    return a > b ? a : b;
}

typedef struct {
    int mode;
    int qe4m3;  /* the E4M3 query (MO_QE4M3) */
    int psplit; /* P as E4M3 hi + lo (MO_PSPLIT) */
    int splits; /* S >= 1 */
    int chunk;  /* keys per chunk >= 1 */
} mo_plan;

/* x_j before the softmax scale: q . dec(K_j) over all 576 bytes (k_scale applied by the caller). */
static double dot_qk(const double* qd, const uint8_t* krow)
{
    double acc = 0.0;
    for (int c = 0; c < MO_ROW; c++)
        acc += qd[c] * mo_e4m3_decode(krow[c]);
    return acc;
}

/*
 * One query row against its group's ordered key list.
 *   keyrow[j]  cache row of key j (j < n_group), or -1 when the key is absent;
 *   n_visible  keys [0, n_visible) may be seen by this row (causal bound), n_visible <= n_group;
 *   starts     NULL: plan->splits splits of per = ceil(n_group / splits) keys each; else nstart
 *              split start keys (starts[0] = 0, non-decreasing, <= n_group), split s ending where
 *              split s + 1 starts (the last at n_group).
 * Writes o[512] and *lse.
 */
static void row_eval(const uint16_t* q, const uint8_t* kv, const int64_t* keyrow, int n_group,
                     int n_visible, double scale, double k_scale, const mo_plan* plan,
                     const int64_t* starts, int nstart, double* o, double* lse, double* amb)
{
    if (amb)
        for (int c = 0; c < MO_LATENT; c++)
            amb[c] = 0.0;
    double qd[MO_ROW];
    for (int c = 0; c < MO_ROW; c++)
        qd[c] = mo_bf16_decode(q[c]);
    if (plan->qe4m3) {
        double qe[MO_ROW];
        mo_q_e4m3(qd, qe);
        memcpy(qd, qe, sizeof qd);
    }
    for (int c = 0; c < MO_LATENT; c++)
        o[c] = 0.0;

    if (plan->mode == MO_EXACT) {
        /* textbook softmax over the visible, present keys */
        double xmax = -INFINITY;
        int any = 0;
        double* x = (double*)malloc(sizeof(double) * (n_visible > 0 ? n_visible : 1));
        for (int j = 0; j < n_visible; j++) {
            if (keyrow[j] < 0)
                continue;
            const uint8_t* kr = kv + (size_t)keyrow[j] * MO_ROW;
            double qk = 0.0;
            for (int c = 0; c < MO_ROW; c++)
                qk += qd[c] * (k_scale * mo_e4m3_decode(kr[c]));
            x[j] = scale * qk;
            if (x[j] > xmax)
                xmax = x[j];
            any = 1;
        }
        if (!any) {
            *lse = -INFINITY;
            free(x);
            return;
        }
        double z = 0.0;
        for (int j = 0; j < n_visible; j++) {
            if (keyrow[j] < 0)
                continue;
            const uint8_t* vr = kv + (size_t)keyrow[j] * MO_ROW;
            double w = exp(x[j] - xmax);
            z += w;
            for (int c = 0; c < MO_LATENT; c++)
                o[c] += w * (k_scale * mo_e4m3_decode(vr[c]));
        }
        for (int c = 0; c < MO_LATENT; c++)
            o[c] /= z;
        *lse = xmax + log(z);
        free(x);
        return;
    }

    /* The split / chunked online softmax (MO_ONLINE, MO_METHOD), logits in log2 units. */
    const int want_amb = amb && plan->mode == MO_METHOD;
    mo_qsplit* qs = want_amb ? (mo_qsplit*)malloc(sizeof(mo_qsplit)) : NULL;
    if (qs)
        split_query(q, plan->qe4m3, scale, k_scale, qs);
    const double log2e = 1.0 / log(2.0);
    const double anchor = 448.0;
    const int S = starts ? nstart : plan->splits;
    double* m_s = (double*)malloc(sizeof(double) * S);
    double* l_s = (double*)malloc(sizeof(double) * S);
    double* O_s = (double*)calloc((size_t)S * MO_LATENT, sizeof(double));
    double* A_s = (double*)calloc((size_t)S * MO_LATENT, sizeof(double)); /* allowance */
    double* x2 = (double*)malloc(sizeof(double) * (plan->chunk > 0 ? plan->chunk : 1));
    double* p = (double*)malloc(sizeof(double) * (plan->chunk > 0 ? plan->chunk : 1));
    double* dx = (double*)malloc(sizeof(double) * (plan->chunk > 0 ? plan->chunk : 1));

    int n = n_group;
    int per = (n + S - 1) / S;
    for (int s = 0; s < S; s++) {
        int first, mine;
        if (starts) {
            first = (int)starts[s];
            mine = (int)((s + 1 < S ? starts[s + 1] : n) - first);
        } else {
            first = s * per < n ? s * per : n;
            mine = n - first < per ? n - first : per;
        }
        double m = -INFINITY, l = 0.0;
        double dm = 0.0; /* d(m): the largest bound among the keys of the part so far */
        double* O = O_s + (size_t)s * MO_LATENT;
        double* A = A_s + (size_t)s * MO_LATENT;
        for (int base = first; base < first + mine; base += plan->chunk) {
            int count = first + mine - base < plan->chunk ? first + mine - base : plan->chunk;
            /* logits of the chunk; -inf for keys the row may not see or that are absent */
            double cmax = -INFINITY;
            for (int t = 0; t < count; t++) {
                int j = base + t;
                if (j >= n_visible || keyrow[j] < 0) {
                    x2[t] = -INFINITY;
                    continue;
                }
                const uint8_t* kr = kv + (size_t)keyrow[j] * MO_ROW;
                x2[t] = scale * k_scale * dot_qk(qd, kr) * log2e;
                if (x2[t] > cmax)
                    cmax = x2[t];
                if (qs) {
                    dx[t] = logit_error_bound(qs, kr) + ldexp(fabs(x2[t]), -23);
                    if (dx[t] > dm)
                        dm = dx[t];
                }
            }
            double m_new = m > cmax ? m : cmax;
            if (m_new == -INFINITY)
                continue; /* nothing visible yet: O and l stay zero */
            double alpha = (m == -INFINITY) ? 1.0 : exp2(m - m_new);
            /* P anchored at 448 of the running maximum; the row sum takes the unrounded P (FP32 on
             * the pages, FP64 here) */
            double total = 0.0;
            for (int t = 0; t < count; t++) {
                p[t] = (x2[t] == -INFINITY) ? 0.0 : anchor * exp2(x2[t] - m_new);
                total += p[t];
            }
            l = l * alpha + total;
            for (int c = 0; c < MO_LATENT; c++) {
                O[c] *= alpha;
                A[c] *= alpha;
            }
            for (int t = 0; t < count; t++) {
                if (p[t] == 0.0)
                    continue;
                double pq = p[t];
                if (plan->mode == MO_METHOD)
                    pq = mo_p_used(p[t], plan->psplit);
                const uint8_t* vr = kv + (size_t)keyrow[base + t] * MO_ROW;
                for (int c = 0; c < MO_LATENT; c++)
                    O[c] += pq * mo_e4m3_decode(vr[c]);
                double d = 0.0;
                if (qs) {
                    const double rel = exp2(dx[t] + ldexp(fabs(x2[t] - m_new), -23) + dm) - 1.0 +
                                       ldexp(1.0, -22);
                    d = rounding_ambiguity(p[t], plan->psplit, rel);
                }
                if (d > 0.0)
                    for (int c = 0; c < MO_LATENT; c++)
                        A[c] += d * fabs(mo_e4m3_decode(vr[c]));
            }
            m = m_new;
        }
        m_s[s] = m;
        l_s[s] = l;
    }

    /* merge of the splits in split order */
    double top = -INFINITY;
    for (int s = 0; s < S; s++)
        if (m_s[s] > top)
            top = m_s[s];
    if (top == -INFINITY) {
        *lse = -INFINITY;
    } else {
        double total = 0.0;
        for (int s = 0; s < S; s++) {
            double w = (m_s[s] == -INFINITY) ? 0.0 : exp2(m_s[s] - top);
            total += w * l_s[s];
            for (int c = 0; c < MO_LATENT; c++) {
                o[c] += w * O_s[(size_t)s * MO_LATENT + c];
                if (amb)
                    amb[c] += w * A_s[(size_t)s * MO_LATENT + c];
            }
        }
        for (int c = 0; c < MO_LATENT; c++) {
            o[c] = o[c] * k_scale / total;
            if (amb)
                amb[c] = amb[c] * k_scale / total;
        }
        *lse = (top - log2(anchor) + log2(total)) * log(2.0);
    }
    free(m_s);
    free(l_s);
    free(O_s);
    free(A_s);
    free(x2);
    free(p);
    free(dx);
    free(qs);
}

/* ---- dense (paged) and sparse (index list) front ends ------------------------------------------ */

typedef struct {
    int dense;
    const uint16_t* q;
    int B, Q, H;
    const uint8_t* kv;
    int64_t num_rows;
    int page_size;
    const int32_t* table;
    int max_pages;
    const int32_t* seq_lens;
    const int32_t* rows;
    int K;
    const int32_t* valid;
    double scale, k_scale;
    mo_plan plan;
    const int64_t* cut_ptr;   /* [groups + 1] or NULL; group g's split starts are */
    const int64_t* cut_start; /* cut_start[cut_ptr[g] .. cut_ptr[g + 1]) */
    const int64_t* sel;
    int64_t n_items;
    double* o;
    double* lse;
    double* amb;   /* optional [items, 512] */
    int nthreads;
    int tid;
} mo_job;

static int clampi(long long v, long long lo, long long hi)
{
    return (int)(v < lo ? lo : (v > hi ? hi : v));
}

static void eval_item(const mo_job* jb, int64_t item)
{
    int64_t flat = jb->sel ? jb->sel[item] : item; /* (b * Q + i) * H + h */
    int i = (int)((flat / jb->H) % jb->Q);
    int b = (int)(flat / ((int64_t)jb->H * jb->Q));
    const uint16_t* q = jb->q + (size_t)flat * MO_ROW;
    int n_group, n_visible;
    int64_t* keyrow;
    if (jb->dense) {
        long long cap = (long long)jb->max_pages * jb->page_size;
        n_group = clampi(jb->seq_lens[b], 0, cap);
        n_visible = clampi((long long)n_group - jb->Q + i + 1, 0, n_group);
        keyrow = (int64_t*)malloc(sizeof(int64_t) * (n_group > 0 ? n_group : 1));
        for (int j = 0; j < n_group; j++) {
            int32_t page = jb->table[(size_t)b * jb->max_pages + j / jb->page_size];
            int64_t r = (int64_t)page * jb->page_size + j % jb->page_size;
            keyrow[j] = (page >= 0 && r < jb->num_rows) ? r : -1;
        }
    } else {
        n_group = clampi(jb->valid[(size_t)b * jb->Q + i], 0, jb->K);
        n_visible = n_group;
        keyrow = (int64_t*)malloc(sizeof(int64_t) * (n_group > 0 ? n_group : 1));
        for (int j = 0; j < n_group; j++) {
            int32_t r = jb->rows[((size_t)b * jb->Q + i) * jb->K + j];
            keyrow[j] = (r >= 0 && r < jb->num_rows) ? r : -1;
        }
    }
    const int64_t g = jb->dense ? b : (int64_t)b * jb->Q + i;
    const int64_t* starts = jb->cut_ptr ? jb->cut_start + jb->cut_ptr[g] : NULL;
    const int nstart = jb->cut_ptr ? (int)(jb->cut_ptr[g + 1] - jb->cut_ptr[g]) : 0;
    row_eval(q, jb->kv, keyrow, n_group, n_visible, jb->scale, jb->k_scale, &jb->plan, starts,
             nstart, jb->o + (size_t)item * MO_LATENT, jb->lse + item,
             jb->amb ? jb->amb + (size_t)item * MO_LATENT : NULL);
    free(keyrow);
}

static void* worker(void* arg)
{
    const mo_job* jb = (const mo_job*)arg;
    for (int64_t it = jb->tid; it < jb->n_items; it += jb->nthreads)
        eval_item(jb, it);
    return NULL;
}

/* Explicit split boundaries must cover each group's keys: at least one split, the first at key 0,
 * non-decreasing starts, none past the group's key count. */
static int check_cuts(const mo_job* jb)
{
    if (!jb->cut_ptr)
        return 0;
    const int64_t groups = jb->dense ? jb->B : (int64_t)jb->B * jb->Q;
    for (int64_t g = 0; g < groups; g++) {
        int n;
        if (jb->dense)
            n = clampi(jb->seq_lens[g], 0, (long long)jb->max_pages * jb->page_size);
        else
            n = clampi(jb->valid[g], 0, jb->K);
        const int64_t a = jb->cut_ptr[g], e = jb->cut_ptr[g + 1];
        if (e <= a || jb->cut_start[a] != 0)
            return -1;
        for (int64_t k = a; k < e; k++)
            if (jb->cut_start[k] > n || (k > a && jb->cut_start[k] < jb->cut_start[k - 1]))
                return -1;
    }
    return 0;
}

static int run_job(mo_job* base)
{
    int nt = base->nthreads < 1 ? 1 : base->nthreads;
    if (base->plan.mode != MO_EXACT && (base->plan.splits < 1 || base->plan.chunk < 1))
        return -1;
    if (check_cuts(base) != 0)
        return -1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nt);
    mo_job* jobs = (mo_job*)malloc(sizeof(mo_job) * nt);
    for (int t = 0; t < nt; t++) {
        jobs[t] = *base;
        jobs[t].nthreads = nt;
        jobs[t].tid = t;
        pthread_create(&th[t], NULL, worker, &jobs[t]);
    }
    for (int t = 0; t < nt; t++)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return 0;
}

/*
 * Dense paged decode. q [B,Q,H,576] bf16 bits; kv [num_rows,576] E4M3 bytes; table [B,max_pages];
 * seq_lens [B]. sel: optional list of flat rows (b*Q+i)*H+h (n_sel of them); NULL means every row.
 * cut_ptr / cut_start: optional explicit split starts per key group (dense: group b; sparse: group
 * b*Q+i), which replace the uniform split rule when given.
 * mode: MO_EXACT, MO_ONLINE or MO_METHOD, plus MO_QE4M3 for the E4M3 query and (METHOD only)
 * MO_PSPLIT for P as E4M3 hi + lo.
 * o [items,512] and lse [items] in FP64; amb (optional, METHOD mode) [items,512] the rounding
 * allowance described at the top.
 */
int mo_dense(const uint16_t* q, int B, int Q, int H, const uint8_t* kv, int64_t num_rows,
             int page_size, float k_scale, const int32_t* table, int max_pages,
             const int32_t* seq_lens, float scale, int mode, int splits, int chunk,
             const int64_t* cut_ptr, const int64_t* cut_start, const int64_t* sel, int64_t n_sel,
             int threads, double* o, double* lse, double* amb)
{
    if (page_size < 1)
        return -1;
    mo_job jb = {0};
    jb.dense = 1;
    jb.q = q;
    jb.B = B;
    jb.Q = Q;
    jb.H = H;
    jb.kv = kv;
    jb.num_rows = num_rows;
    jb.page_size = page_size;
    jb.table = table;
    jb.max_pages = max_pages;
    jb.seq_lens = seq_lens;
    jb.scale = scale;
    jb.k_scale = k_scale;
    jb.plan.mode = mode & ~(MO_QE4M3 | MO_PSPLIT);
    jb.plan.qe4m3 = (mode & MO_QE4M3) != 0;
    jb.plan.psplit = (mode & MO_PSPLIT) != 0;
    jb.plan.splits = splits;
    jb.plan.chunk = chunk;
    jb.cut_ptr = cut_ptr;
    jb.cut_start = cut_start;
    jb.sel = sel;
    jb.n_items = sel ? n_sel : (int64_t)B * Q * H;
    jb.o = o;
    jb.lse = lse;
    jb.amb = amb;
    jb.nthreads = threads;
    return run_job(&jb);
}

/*
 * Sparse (top-k list) decode. rows [B,Q,K] flat cache rows, valid [B,Q] counts (clamped to [0,K]).
 */
int mo_sparse(const uint16_t* q, int B, int Q, int H, const uint8_t* kv, int64_t num_rows,
              float k_scale, const int32_t* rows, int K, const int32_t* valid, float scale,
              int mode, int splits, int chunk, const int64_t* cut_ptr, const int64_t* cut_start,
              const int64_t* sel, int64_t n_sel, int threads, double* o, double* lse, double* amb)
{
    mo_job jb = {0};
    jb.dense = 0;
    jb.q = q;
    jb.B = B;
    jb.Q = Q;
    jb.H = H;
    jb.kv = kv;
    jb.num_rows = num_rows;
    jb.rows = rows;
    jb.K = K;
    jb.valid = valid;
    jb.scale = scale;
    jb.k_scale = k_scale;
    jb.plan.mode = mode & ~(MO_QE4M3 | MO_PSPLIT);
    jb.plan.qe4m3 = (mode & MO_QE4M3) != 0;
    jb.plan.psplit = (mode & MO_PSPLIT) != 0;
    jb.plan.splits = splits;
    jb.plan.chunk = chunk;
    jb.cut_ptr = cut_ptr;
    jb.cut_start = cut_start;
    jb.sel = sel;
    jb.n_items = sel ? n_sel : (int64_t)B * Q * H;
    jb.o = o;
    jb.lse = lse;
    jb.amb = amb;
    jb.nthreads = threads;
    return run_job(&jb);
}

/* ---- combine of partial decodes (decode-context parallel merge) ------------------------------ */

/*
 * R partial results of the same query rows, each over a disjoint part of the rows' keys (a rank's
 * share), merged the way the split partials are ([SPARSE] module docstring and merge: weights
 * exp2(m_s - top), divided by the weighted total), here with natural-log LSEs, in rank order:
 *   M = max_r lse_r;  w_r = exp(lse_r - M), 0 where lse_r = -inf;  L = sum_r w_r;
 *   o = sum_r w_r o_r / L;  lse = M + ln L.
 * A row with no partial holding a key (every lse_r = -inf) gets o = +0 and lse = -inf. A partial
 * with lse_r = -inf is skipped without reading its o row (the page's push mode sends only the LSE
 * of such a row).
 * o_parts [R, rows, 512], lse_parts [R, rows]; o [rows, 512], lse [rows].
 */
void mo_combine_f64(const double* o_parts, const double* lse_parts, int R, int64_t rows, double* o,
                    double* lse)
{
    for (int64_t i = 0; i < rows; i++) {
        double M = -INFINITY;
        for (int r = 0; r < R; r++)
            if (lse_parts[(size_t)r * rows + i] > M)
                M = lse_parts[(size_t)r * rows + i];
        double* oi = o + (size_t)i * MO_LATENT;
        for (int c = 0; c < MO_LATENT; c++)
            oi[c] = 0.0;
        if (M == -INFINITY) {
            lse[i] = -INFINITY;
            continue;
        }
        double L = 0.0;
        for (int r = 0; r < R; r++) {
            const double l = lse_parts[(size_t)r * rows + i];
            if (l == -INFINITY)
                continue; /* a rank without keys sends only its LSE: its o row is not read */
            const double w = exp(l - M);
            L += w;
            const double* orow = o_parts + ((size_t)r * rows + i) * MO_LATENT;
            for (int c = 0; c < MO_LATENT; c++)
                oi[c] += w * orow[c];
        }
        for (int c = 0; c < MO_LATENT; c++)
            oi[c] /= L;
        lse[i] = M + log(L);
    }
}

/* The same from the decode's output formats: o_parts bf16 bits, lse_parts FP32 (both exact in
 * FP64). */
void mo_combine(const uint16_t* o_parts, const float* lse_parts, int R, int64_t rows, double* o,
                double* lse)
{
    const size_t n = (size_t)R * rows;
    double* od = (double*)malloc(sizeof(double) * n * MO_LATENT + 1);
    double* ld = (double*)malloc(sizeof(double) * n + 1);
    for (size_t k = 0; k < n * MO_LATENT; k++)
        od[k] = mo_bf16_decode(o_parts[k]);
    for (size_t k = 0; k < n; k++)
        ld[k] = (double)lse_parts[k];
    mo_combine_f64(od, ld, R, rows, o, lse);
    free(od);
    free(ld);
}
