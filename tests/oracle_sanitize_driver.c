/*
 * Driver of the oracle library (oracle/mla_oracle.c) for a host build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point on small seeded inputs, with the edge cases the
 * oracle handles (empty and clamped counts, absent keys, keys before the causal bound, explicit
 * split starts, row selections, all precision flags, the allowance), plus two checks that make a
 * run meaningful beyond the sanitizers: the ONLINE mode equals EXACT for every plan (the split
 * identity) and every output is finite or an empty row's -inf. Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mo_dense(const uint16_t* q, int B, int Q, int H, const uint8_t* kv, int64_t num_rows,
             int page_size, float k_scale, const int32_t* table, int max_pages,
             const int32_t* seq_lens, float scale, int mode, int splits, int chunk,
             const int64_t* cut_ptr, const int64_t* cut_start, const int64_t* sel, int64_t n_sel,
             int threads, double* o, double* lse, double* amb);
int mo_sparse(const uint16_t* q, int B, int Q, int H, const uint8_t* kv, int64_t num_rows,
              float k_scale, const int32_t* rows, int K, const int32_t* valid, float scale,
              int mode, int splits, int chunk, const int64_t* cut_ptr, const int64_t* cut_start,
              const int64_t* sel, int64_t n_sel, int threads, double* o, double* lse, double* amb);
void mo_combine(const uint16_t* o_parts, const float* lse_parts, int R, int64_t rows, double* o,
                double* lse);
double mo_e4m3_decode(uint8_t c);
uint8_t mo_e4m3_encode(double x);
double mo_p_used(double p, int split);
void mo_q_e4m3_bits(const uint16_t* q, double* qe);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t rnd(void)
{   /* xorshift64* (Vigna 2016) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* a bf16 pattern of a value of modest size (sign, exponent 120..130, random mantissa) */
static uint16_t rnd_bf16(void)
{
    const uint32_t s = rnd() & 1u, e = 120u + rnd() % 11u, m = rnd() & 0x7Fu;
    return (uint16_t)((s << 15) | (e << 7) | m);
}

/* an E4M3 code that is not NaN */
static uint8_t rnd_e4m3(void)
{
    uint8_t c;
    do
        c = (uint8_t)rnd();
    while ((c & 0x7F) == 0x7F);
    return c;
}

static int failures = 0;

static void expect(int ok, const char* what)
{
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        failures++;
    }
}

static void check_outputs(const double* o, const double* lse, int64_t n, const char* what)
{
    for (int64_t r = 0; r < n; r++) {
        if (isinf(lse[r]) && lse[r] < 0) {
            for (int c = 0; c < 512; c++)
                expect(o[r * 512 + c] == 0.0 && !signbit(o[r * 512 + c]), what);
            continue;
        }
        expect(isfinite(lse[r]), what);
        for (int c = 0; c < 512; c++)
            expect(isfinite(o[r * 512 + c]), what);
    }
}

static void check_close(const double* a, const double* b, int64_t n, double tol, const char* what)
{
    for (int64_t k = 0; k < n; k++) {
        if (isinf(a[k]) || isinf(b[k])) {
            expect(a[k] == b[k], what);
            continue;
        }
        expect(fabs(a[k] - b[k]) <= tol * (1.0 + fabs(b[k])), what);
    }
}

int main(void)
{
    const int B = 3, Q = 2, H = 2, page = 8, max_pages = 6, num_rows = 64;
    const int rows_q = B * Q * H;
    uint16_t* q = malloc(sizeof(uint16_t) * rows_q * 576);
    uint8_t* kv = malloc((size_t)num_rows * 576);
    for (int k = 0; k < rows_q * 576; k++)
        q[k] = rnd_bf16();
    for (int k = 0; k < num_rows * 576; k++)
        kv[k] = rnd_e4m3();
    /* dense: a table with an absent page (id past the pool) and an unused tail */
    int32_t table[3 * 6];
    for (int k = 0; k < B * max_pages; k++)
        table[k] = (int32_t)(rnd() % 8u);
    table[1 * max_pages + 2] = 1000;
    const int32_t seq[3] = {37, 1, 48};   /* 48 = the table's capacity; 1 < Q: rows before the bound */
    double* o = malloc(sizeof(double) * rows_q * 512);
    double* o2 = malloc(sizeof(double) * rows_q * 512);
    double* amb = malloc(sizeof(double) * rows_q * 512);
    double lse[12], lse2[12];
    const float scale = 0.0721687836f, k_scale = 0.05f;

    for (int flags = 0; flags <= 16; flags += 16) {
        expect(mo_dense(q, B, Q, H, kv, num_rows, page, k_scale, table, max_pages, seq, scale,
                        0 | flags, 1, 1, NULL, NULL, NULL, 0, 2, o, lse, NULL) == 0, "dense exact");
        check_outputs(o, lse, rows_q, "dense exact outputs");
        const int plans[4][2] = {{1, 128}, {3, 5}, {7, 1}, {2, 16}};
        for (int p = 0; p < 4; p++) {
            expect(mo_dense(q, B, Q, H, kv, num_rows, page, k_scale, table, max_pages, seq, scale,
                            1 | flags, plans[p][0], plans[p][1], NULL, NULL, NULL, 0, 3, o2, lse2,
                            NULL) == 0, "dense online");
            check_close(o2, o, (int64_t)rows_q * 512, 1e-9, "online == exact (o)");
            check_close(lse2, lse, rows_q, 1e-12, "online == exact (lse)");
            for (int ps = 0; ps <= 32; ps += 32) {
                expect(mo_dense(q, B, Q, H, kv, num_rows, page, k_scale, table, max_pages, seq,
                                scale, 2 | flags | ps, plans[p][0], plans[p][1], NULL, NULL, NULL,
                                0, 2, o2, lse2, amb) == 0, "dense method");
                check_outputs(o2, lse2, rows_q, "dense method outputs");
                check_close(lse2, lse, rows_q, 1e-12, "method lse == exact lse");
            }
        }
    }
    /* explicit split starts (one group has none past 0, one is cut at its end) and a selection */
    const int64_t cut_ptr[4] = {0, 3, 4, 6};
    const int64_t cut_start[6] = {0, 8, 37, 0, 0, 48};
    const int64_t sel[5] = {0, 3, 5, 11, 6};
    expect(mo_dense(q, B, Q, H, kv, num_rows, page, k_scale, table, max_pages, seq, scale, 2, 1,
                    4, cut_ptr, cut_start, sel, 5, 2, o2, lse2, amb) == 0, "dense cuts + sel");
    check_outputs(o2, lse2, 5, "dense cuts + sel outputs");
    const int64_t bad_start[6] = {1, 8, 37, 0, 0, 48};
    expect(mo_dense(q, B, Q, H, kv, num_rows, page, k_scale, table, max_pages, seq, scale, 2, 1,
                    4, cut_ptr, bad_start, NULL, 0, 1, o2, lse2, NULL) != 0, "bad cuts refused");

    /* sparse: counts past K and negative, absent and duplicate indices */
    const int K = 20;
    int32_t* rows = malloc(sizeof(int32_t) * B * Q * K);
    for (int k = 0; k < B * Q * K; k++)
        rows[k] = (int32_t)(rnd() % (unsigned)num_rows);
    rows[3] = -1;
    rows[K + 1] = num_rows;
    rows[2 * K] = rows[2 * K + 1];
    const int32_t valid[6] = {20, 500, -4, 0, 1, 13};
    expect(mo_sparse(q, B, Q, H, kv, num_rows, k_scale, rows, K, valid, scale, 0, 1, 1, NULL, NULL,
                     NULL, 0, 2, o, lse, NULL) == 0, "sparse exact");
    check_outputs(o, lse, rows_q, "sparse exact outputs");
    for (int mode = 1; mode <= 2; mode++) {
        expect(mo_sparse(q, B, Q, H, kv, num_rows, k_scale, rows, K, valid, scale, mode, 4, 3,
                         NULL, NULL, NULL, 0, 2, o2, lse2, mode == 2 ? amb : NULL) == 0,
               "sparse online / method");
        check_outputs(o2, lse2, rows_q, "sparse outputs");
        check_close(lse2, lse, rows_q, 1e-12, "sparse lse");
        if (mode == 1)
            check_close(o2, o, (int64_t)rows_q * 512, 1e-9, "sparse online == exact");
    }

    /* combine of three ranks' bf16 rows, one rank empty for some rows (its o rows NaN) */
    const int R = 3, crow = 7;
    uint16_t* parts = malloc(sizeof(uint16_t) * R * crow * 512);
    float lparts[21];
    for (int k = 0; k < R * crow * 512; k++)
        parts[k] = rnd_bf16();
    for (int k = 0; k < R * crow; k++)
        lparts[k] = (float)((int)(rnd() % 200u) - 100) / 10.0f;
    for (int r = 0; r < crow; r += 2) {
        lparts[crow + r] = -INFINITY;
        for (int c = 0; c < 512; c++)
            parts[((size_t)crow + r) * 512 + c] = 0x7FC0;
    }
    for (int r = 0; r < R; r++)
        lparts[r * crow + 3] = -INFINITY;   /* row 3: no rank holds a key */
    mo_combine(parts, lparts, R, crow, o, lse);
    check_outputs(o, lse, crow, "combine outputs");
    expect(isinf(lse[3]) && lse[3] < 0, "combine empty row");

    /* the codecs over their whole domains */
    for (int c = 0; c < 256; c++) {
        const double v = mo_e4m3_decode((uint8_t)c);
        if (!isnan(v))
            expect(mo_e4m3_encode(v) == (uint8_t)c || (v == 0.0), "e4m3 round trip");
    }
    for (int k = 0; k < 4096; k++) {
        const double p = ldexp(1.0 + (rnd() % 1000u) / 1000.0, (int)(rnd() % 20u) - 12);
        expect(fabs(mo_p_used(p, 1) - p) <= fmax(ldexp(p, -8), ldexp(1.0, -10)) * 1.0001,
               "p split bound");
    }
    double qe[576];
    mo_q_e4m3_bits(q, qe);
    for (int c = 0; c < 576; c++)
        expect(isfinite(qe[c]), "e4m3 query");

    free(q);
    free(kv);
    free(o);
    free(o2);
    free(amb);
    free(rows);
    free(parts);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
