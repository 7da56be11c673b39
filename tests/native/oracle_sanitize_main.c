/* Drives the C routing oracle (oracle/route_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: exp and the pairwise sum over their argument ranges, the
 * softmax up to 256 experts, the capacity helper, and full routings (dropless, drops per
 * sub-sequence, capacity 0, exact ties, K = E, 256 experts, empty input, rejected
 * arguments), each checked for the invariants of the maps.  Exit 0 and "ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

float oracle_exp(float r);
float oracle_pairwise_sum(const float* v, int n);
void oracle_softmax_row(const float* logit, int E, float* p);
int oracle_capacity(int S, int K, int E, double cf);
int oracle_route(int T, int E, int K, int S, int capacity, const float* logits,
                 int32_t* topk_idx, float* topk_prob, float* topk_gate, uint8_t* keep,
                 int32_t* row_of, int32_t* src_of, int32_t* routed_counts,
                 int32_t* kept_counts, int32_t* offsets, int32_t* n_kept);

static uint64_t g_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
    g_state ^= g_state << 13; g_state ^= g_state >> 7; g_state ^= g_state << 17;
    return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}

#define CHECK(c, ...) do { if (!(c)) { printf("FAIL: " __VA_ARGS__); printf("\n"); exit(1); } } while (0)

static void route_case(int T, int E, int K, int S, int cap, int ties) {
    const size_t TK = (size_t)T * K;
    float* lg = malloc(sizeof(float) * ((size_t)T * E + 1));
    for (size_t i = 0; i < (size_t)T * E; ++i)
        lg[i] = ties ? (float)(int)(urand() * 4.0) : (float)(4.0 * (urand() - 0.5));
    int32_t* idx = malloc(sizeof(int32_t) * (TK + 1));
    float* prob = malloc(sizeof(float) * (TK + 1));
    float* gate = malloc(sizeof(float) * (TK + 1));
    uint8_t* keep = malloc(TK + 1);
    int32_t* row = malloc(sizeof(int32_t) * (TK + 1));
    int32_t* src = malloc(sizeof(int32_t) * (TK + 1));
    int n_sub = T / S;
    int32_t* rc = malloc(sizeof(int32_t) * ((size_t)(n_sub ? n_sub : 1) * E));
    int32_t* kc = malloc(sizeof(int32_t) * E);
    int32_t* off = malloc(sizeof(int32_t) * (E + 1));
    int32_t nk = -1;
    CHECK(oracle_route(T, E, K, S, cap, lg, idx, prob, gate, keep, row, src, rc, kc, off, &nk) == 0,
          "route T=%d E=%d K=%d S=%d cap=%d", T, E, K, S, cap);
    CHECK(off[0] == 0 && off[E] == nk, "offsets");
    long kept = 0;
    for (int e = 0; e < E; ++e) {
        CHECK(off[e + 1] - off[e] == kc[e] && kc[e] >= 0, "kept counts");
        for (int s = 0; s < n_sub; ++s) CHECK(cap < 0 || kc[e] <= (long)n_sub * cap, "capacity");
    }
    for (int t = 0; t < T; ++t) {
        float gs = 0.0f;
        for (int k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            CHECK(idx[i] >= 0 && idx[i] < E, "expert index");
            CHECK(k == 0 || prob[i - 1] > prob[i] || (prob[i - 1] == prob[i] && idx[i - 1] < idx[i]),
                  "slot order");
            gs += gate[i];
            if (keep[i]) {
                ++kept;
                CHECK(row[i] >= off[idx[i]] && row[i] < off[idx[i] + 1], "row in its segment");
                CHECK(src[row[i]] == (int32_t)i, "src_of inverts row_of");
            } else {
                CHECK(row[i] == -1, "dropped row");
            }
        }
        CHECK(fabsf(gs - 1.0f) <= 1e-5f, "gates sum to 1");
    }
    CHECK(kept == nk, "n_kept");
    free(lg); free(idx); free(prob); free(gate); free(keep); free(row); free(src); free(rc);
    free(kc); free(off);
}

int main(void) {
    for (int i = 0; i < 200000; ++i) {
        float r = (float)(-100.0 * urand());
        float y = oracle_exp(r);
        CHECK(y >= 0.0f && y <= 1.0f && isfinite(y), "exp(%g)", (double)r);
    }
    CHECK(oracle_exp(0.0f) == 1.0f, "exp(0)");
    float v[300];
    for (int i = 0; i < 300; ++i) v[i] = (float)i;
    for (int n = 1; n <= 256; ++n) CHECK(oracle_pairwise_sum(v, n) == (float)(n * (n - 1) / 2), "sum %d", n);
    CHECK(oracle_pairwise_sum(v, 0) == 0.0f && oracle_pairwise_sum(v, 257) == 0.0f, "sum range");
    float p[256];
    for (int E = 1; E <= 256; E *= 2) {
        for (int e = 0; e < E; ++e) v[e] = (float)(urand() * 10.0 - 5.0);
        oracle_softmax_row(v, E, p);
        double s = 0.0;
        for (int e = 0; e < E; ++e) s += p[e];
        CHECK(fabs(s - 1.0) < 1e-5, "softmax E=%d", E);
    }
    CHECK(oracle_capacity(4096, 2, 8, 1.0) == 1024 && oracle_capacity(8, 2, 4, -1.0) == -1, "capacity");
    route_case(0, 4, 2, 1, -1, 0);
    route_case(256, 4, 2, 256, -1, 0);
    route_case(1024, 8, 2, 256, 64, 0);
    route_case(1024, 8, 2, 256, 64, 1);
    route_case(512, 64, 8, 512, 0, 0);
    route_case(600, 3, 3, 200, 10, 1);
    route_case(100, 256, 8, 50, 2, 0);
    route_case(96, 16, 4, 32, 1000, 1);
    int32_t dummy[64];
    float fd[64];
    uint8_t ud[64];
    CHECK(oracle_route(10, 4, 2, 3, -1, fd, dummy, fd, fd, ud, dummy, dummy, dummy, dummy, dummy,
                       dummy) == -1, "T %% S rejected");
    CHECK(oracle_route(8, 4, 5, 8, -1, fd, dummy, fd, fd, ud, dummy, dummy, dummy, dummy, dummy,
                       dummy) == -1, "K > E rejected");
    CHECK(oracle_route(8, 257, 1, 8, -1, fd, dummy, fd, fd, ud, dummy, dummy, dummy, dummy, dummy,
                       dummy) == -1, "E > 256 rejected");
    printf("ok\n");
    return 0;
}
