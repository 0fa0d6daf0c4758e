/*
 * Sanitizer check program for the C oracle (oracle/mla_oracle.c), built by
 * tests/test_sanitizers.py with AddressSanitizer and UndefinedBehaviorSanitizer
 * and linked against the oracle's source.  Every array is allocated at its
 * exact size, so an access one element past any of them is reported.  It
 * calls each oracle function on small seeded inputs, including padding (-1),
 * repeated indices, an empty selection and ragged lengths, and checks the
 * status codes and that each softmax row sums to one.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_decode(int64_t B, int64_t H, int64_t Dn, int64_t Dc, int64_t Dr, int64_t Dv, const double* q_nope,
                  const double* q_pe, const double* kv, int64_t kv_sb, int64_t kv_st, const double* pe, int64_t pe_sb,
                  int64_t pe_st, const double* wkv_b, const int32_t* seq_lens, const int64_t* indices, int64_t k_max,
                  double scale, double* q_abs, double* o_lat, double* out, double* lse, unsigned char* attended,
                  int64_t att_stride, double* weights, double* scores);
int oracle_prefill(int64_t B, int64_t T, int64_t H, int64_t Dn, int64_t Dc, int64_t Dr, int64_t Dv,
                   const double* q_nope, const double* q_pe, const double* kv, int64_t kv_sb, int64_t kv_st,
                   const double* pe, int64_t pe_sb, int64_t pe_st, const double* wkv_b, const int64_t* indices,
                   int64_t k_max, double scale, double* out, double* lse, unsigned char* attended);
int oracle_absorb(int64_t B, int64_t H, int64_t Dn, int64_t Dc, int64_t Dv, const double* q_nope,
                  const double* wkv_b, double* q_abs);
int oracle_value_up(int64_t B, int64_t H, int64_t Dn, int64_t Dc, int64_t Dv, const double* o_lat,
                    const double* wkv_b, double* out);
int oracle_output_proj(int64_t B, int64_t Din, int64_t Dout, const double* x, const double* wo, double* out);
int oracle_dequant_fp8(const uint8_t* w, const float* scales, int64_t rows, int64_t cols, int64_t blk,
                       uint16_t* out_bf16, double* out_exact);

static uint64_t state = 12345;
static double rnd(void) {
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((double)(state >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}
/* Every block this program allocates, freed at the end so that leak
 * detection reports only the oracle's own allocations. */
static void* blocks[64];
static int nblocks = 0;
static void* take(size_t bytes) {
    void* p = malloc(bytes);
    blocks[nblocks++] = p;
    return p;
}
static double* arr(int64_t n) {
    double* p = (double*)take(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
    const int64_t B = 3, H = 4, Dn = 8, Dc = 16, Dr = 4, Dv = 8, L = 9, K = 6;
    double *qn = arr(B * H * Dn), *qr = arr(B * H * Dr), *kv = arr(B * L * Dc), *pe = arr(B * L * Dr);
    double* w = arr(H * (Dn + Dv) * Dc);
    int32_t lens[3] = {9, 5, 7};
    /* row 0: distinct + padding; row 1: a repeat; row 2: empty (all padding) */
    int64_t idx[3 * 6] = {8, 0, 3, -1, 2, -1, 4, 1, 4, 0, -1, 2, -1, -1, -1, -1, -1, -1};
    double *qa = arr(B * H * Dc), *ol = arr(B * H * Dc), *out = arr(B * H * Dv), *lse = arr(B * H);
    double *wts = arr(B * H * K), *sc = arr(B * H * K);
    unsigned char* att = (unsigned char*)take((size_t)(B * L));
    int st = oracle_decode(B, H, Dn, Dc, Dr, Dv, qn, qr, kv, L * Dc, Dc, pe, L * Dr, Dr, w, lens, idx, K,
                           0.3, qa, ol, out, lse, att, L, wts, sc);
    CHECK(st == 4); /* the empty row is reported */
    for (int64_t b = 0; b < 2; ++b)
        for (int64_t h = 0; h < H; ++h) {
            double s = 0.0;
            int64_t seen[16] = {0};
            for (int64_t j = 0; j < K; ++j) {
                const int64_t t = idx[b * K + j];
                if (t >= 0 && !seen[t]) { s += wts[(b * H + h) * K + j]; seen[t] = 1; }
            }
            CHECK(fabs(s - 1.0) < 1e-12);
        }
    CHECK(isnan(out[2 * H * Dv]));
    /* dense (no index list), ragged lengths */
    st = oracle_decode(B, H, Dn, Dc, Dr, Dv, qn, qr, kv, L * Dc, Dc, pe, L * Dr, Dr, w, lens, NULL, 0, 0.3,
                       NULL, NULL, out, lse, NULL, 0, NULL, NULL);
    CHECK(st == 0);
    /* an out-of-range index is rejected */
    int64_t bad[3 * 6] = {8, 0, 3, -1, 2, -1, 5, 1, 4, 0, -1, 2, 0, 1, 2, 3, 4, 5};
    st = oracle_decode(B, H, Dn, Dc, Dr, Dv, qn, qr, kv, L * Dc, Dc, pe, L * Dr, Dr, w, lens, bad, K, 0.3,
                       NULL, NULL, out, NULL, NULL, 0, NULL, NULL);
    CHECK(st & 1);
    /* prefill: T = 5 tokens, index rows with later positions and padding */
    const int64_t T = 5, KP = 3;
    double *pqn = arr(B * T * H * Dn), *pqr = arr(B * T * H * Dr), *pkv = arr(B * T * Dc), *ppe = arr(B * T * Dr);
    int64_t* pidx = (int64_t*)take(sizeof(int64_t) * (size_t)(B * T * KP));
    for (int64_t i = 0; i < B * T * KP; ++i) pidx[i] = (i * 7 + 3) % (T + 1) - 1;
    double *pout = arr(B * T * H * Dv), *plse = arr(B * T * H);
    unsigned char* patt = (unsigned char*)take((size_t)(B * T * T));
    st = oracle_prefill(B, T, H, Dn, Dc, Dr, Dv, pqn, pqr, pkv, T * Dc, Dc, ppe, T * Dr, Dr, w, pidx, KP, 0.3,
                        pout, plse, patt);
    CHECK((st & ~4) == 0);
    st = oracle_prefill(B, T, H, Dn, Dc, Dr, Dv, pqn, pqr, pkv, T * Dc, Dc, ppe, T * Dr, Dr, w, NULL, 0, 0.3,
                        pout, plse, NULL);
    CHECK(st == 0);
    CHECK(oracle_absorb(B, H, Dn, Dc, Dv, qn, w, qa) == 0);
    CHECK(oracle_value_up(B, H, Dn, Dc, Dv, ol, w, out) == 0);
    double *x = arr(2 * 12), *wo = arr(7 * 12), *po = arr(2 * 7);
    CHECK(oracle_output_proj(2, 12, 7, x, wo, po) == 0);
    /* fp8: every code, a ragged block grid (rows and cols not multiples of the block) */
    const int64_t R = 300, C = 200, BLK = 128;
    uint8_t* codes = (uint8_t*)take((size_t)(R * C));
    for (int64_t i = 0; i < R * C; ++i) codes[i] = (uint8_t)(i * 7);
    float* scl = (float*)take(sizeof(float) * 3 * 2);
    for (int i = 0; i < 6; ++i) scl[i] = (float)ldexp(1.0 + 0.1 * i, -6);
    uint16_t* b16 = (uint16_t*)take(sizeof(uint16_t) * (size_t)(R * C));
    double* ex = (double*)take(sizeof(double) * (size_t)(R * C));
    CHECK(oracle_dequant_fp8(codes, scl, R, C, BLK, b16, ex) == 0);
    for (int i = 0; i < nblocks; ++i) free(blocks[i]);
    puts("oracle sanitizer check: ok");
    return 0;
}
