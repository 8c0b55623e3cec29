/* oracle_driver.c -- runs every oracle entry point on small seeded inputs, valid and
 * invalid, for the address / undefined-behaviour sanitizer build of the oracle
 * (tests/test_sanitizers.py).  Exit status 0 when every call returned what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_oracle.h"

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 11);
}
static float normal(void) { /* sum of 12 uniforms minus 6: close enough for test logits */
    float s = 0.f;
    for (int i = 0; i < 12; ++i) s += (float)(next_u32() & 0xffffff) / 16777216.f;
    return s - 6.f;
}
static float coin(void) { return (float)((next_u32() & 0xffffff) + 1) / 16777216.f; }

#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                            \
        }                                                        \
    } while (0)

int main(void) {
    const int B = 5, G = 3, R = G + 1, V = 37, N = 9, D = 3;
    float* lg = malloc(sizeof(float) * B * N * V);
    uint16_t* lb = malloc(sizeof(uint16_t) * B * N * V);
    float* q = malloc(sizeof(float) * B * N * V);
    int32_t x[5 * 9], par[5 * 9], tok[5 * 9], acc[5], out[5 * 10], nodes[5 * 9];
    float u[5 * 9], T[5];
    double probs[5 * 10], margin[5], am[5], beta[5 * 3];
    for (int i = 0; i < B * N * V; ++i) {
        lg[i] = 1.5f * normal();
        uint32_t bits;
        memcpy(&bits, &lg[i], 4);
        lb[i] = (uint16_t)(bits >> 16);
        q[i] = (float)exp(normal());
    }
    for (int r = 0; r < B * N; ++r) { /* q rows normalised */
        double s = 0;
        for (int v = 0; v < V; ++v) s += q[(size_t)r * V + v];
        for (int v = 0; v < V; ++v) q[(size_t)r * V + v] = (float)(q[(size_t)r * V + v] / s);
    }
    for (int i = 0; i < B * N; ++i) {
        x[i] = (int32_t)(next_u32() % V);
        u[i] = coin();
    }
    for (int b = 0; b < B; ++b) T[b] = 0.5f + 0.25f * (float)b;
    x[1 * G + 0] = V + 3; /* request 1: a token outside the vocabulary (invalid) */
    T[2] = -1.f;          /* request 2: a bad temperature (invalid) */

    for (int dt = 0; dt < 2; ++dt) {
        const void* L = dt ? (const void*)lb : (const void*)lg;
        CHECK(oracle_verify_greedy(L, dt, x, B, G, V, acc, out) == 0);
        CHECK(acc[1] == -1);
        CHECK(oracle_verify_chain(L, dt, q, x, u, T, B, G, V, acc, out, probs, margin, beta, am) == 0);
        CHECK(acc[1] == -1 && acc[2] == -1);
        for (int b = 0; b < B; ++b) CHECK(acc[b] >= -1 && acc[b] <= G);
        CHECK(oracle_verify_chain(L, dt, q, x, u, T, B, G, V, acc, out, NULL, margin, NULL, NULL) == 0);
        /* a tree per request: root, three children, grandchildren */
        const int tp[9] = {-1, 0, 0, 0, 1, 1, 2, 4, 7};
        for (int b = 0; b < B; ++b)
            for (int i = 0; i < N; ++i) {
                par[b * N + i] = tp[i];
                tok[b * N + i] = i == 0 ? -1 : (int32_t)((b * 7 + i * 5) % V);
            }
        par[3 * N + 5] = 6; /* request 3: a parent after its child (invalid) */
        CHECK(oracle_verify_tree(L, dt, tok, par, u, T, B, N, V, 4, 1, 1.0f, 1.0f, acc, out,
                                 nodes, probs, margin, am) == 0);
        CHECK(acc[3] == -1);
        CHECK(oracle_verify_tree(L, dt, tok, par, NULL, NULL, B, N, V, 4, 0, 1.0f, 1.0f, acc, out,
                                 nodes, NULL, margin, NULL) == 0);
        CHECK(oracle_verify_tree(L, dt, tok, par, u, T, B, N, V, D, 1, 0.3f, 0.7f, acc, out,
                                 nodes, probs, margin, NULL) == 0);
        CHECK(oracle_verify_tree_mss(L, dt, q, tok, par, u, T, B, N, V, 4, acc, out, nodes,
                                     probs, margin, am) == 0);
        int32_t topk[5] = {0, 5, 1, 40, 3};
        float topp[5] = {1.f, 0.9f, 0.5f, 0.95f, 1.f};
        CHECK(oracle_verify_chain_filtered(L, L, dt, x, u, T, topk, topp, B, G, V, acc, out,
                                           probs, margin, am) == 0);
        CHECK(oracle_verify_chain_filtered(L, L, dt, x, u, T, NULL, NULL, B, G, V, acc, out,
                                           NULL, margin, NULL) == 0);
    }
    uint32_t mask[5 * 9 * 1];
    int32_t pos[5 * 9], base[5] = {0, 3, 7, 100, 1};
    CHECK(oracle_tree_mask(par, base, B, N, mask, pos) == 0);
    CHECK(oracle_tree_mask(par, NULL, B, N, mask, NULL) == 0);
    unsigned char kv_tree[5 * 9 * 24], kv_out[5 * 4 * 24];
    for (size_t i = 0; i < sizeof kv_tree; ++i) kv_tree[i] = (unsigned char)i;
    int32_t an[5 * 3] = {1, 4, 7, 2, 6, -1, 0, 0, 0, 3, -1, -1, 1, 5, -1};
    int32_t al[5] = {3, 2, 5, 1, 2}, slots[5 * 4];
    CHECK(oracle_tree_commit_kv(an, al, B, 3, N, kv_tree, kv_out, 24, slots) == 0);
    /* unusable arguments */
    CHECK(oracle_verify_greedy(NULL, 0, x, B, G, V, acc, out) == -1);
    CHECK(oracle_verify_chain(lg, 0, q, x, u, T, B, 0, V, acc, out, probs, margin, NULL, NULL) == -1);
    CHECK(oracle_verify_tree(lg, 0, tok, par, u, T, B, N, V, 0, 1, 1.f, 1.f, acc, out, nodes,
                             probs, margin, NULL) == -1);
    oracle_set_num_threads(1);
    CHECK(oracle_num_threads() >= 1);
    free(lg);
    free(lb);
    free(q);
    printf("oracle driver: all calls checked\n");
    return 0;
}
