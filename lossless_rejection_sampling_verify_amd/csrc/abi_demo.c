/* abi_demo.c -- a plain C consumer of the verify library's C ABI (include/spec_verify.h).
 *
 * Reads a batch from a binary file, runs spec_verify_greedy and spec_verify_chain on the
 * default stream with device buffers it allocates itself, and writes the outputs to a
 * second file.  It shows the calling sequence a C or C++ serving stack uses: query the
 * workspace size, allocate and zero the workspace once, copy the inputs, call, read back.
 *
 * Input  (little endian): int32 B, G, V; fp32 logits [B][G+1][V]; fp32 q [B][G][V];
 *                         int32 greedy drafts [B][G]; int32 sampled drafts [B][G];
 *                         fp32 coins [B][G+1]; fp32 temperature [B].
 * Output: int32 greedy accept_len [B], greedy tokens [B][G+1], chain accept_len [B],
 *         chain tokens [B][G+1]; fp32 chain probs [B][G+1].
 * Exit status 0 on success, 1 on a usage or file error, 2 on a HIP error, 3 on a
 * library status other than SPEC_OK (printed). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "spec_verify.h"

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

#define HIP(x)                                                              \
    do {                                                                    \
        if ((x) != hipSuccess) {                                            \
            fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);   \
            return 2;                                                       \
        }                                                                   \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
        return 1;
    }
    FILE* fi = fopen(argv[1], "rb");
    if (!fi) return 1;
    int32_t dims[3];
    if (!read_all(fi, dims, sizeof dims)) return 1;
    const int B = dims[0], G = dims[1], V = dims[2], R = G + 1;
    if (B < 1 || G < 1 || G > SPEC_MAX_G || V < 1) return 1;
    const size_t nl = (size_t)B * R * V, nq = (size_t)B * G * V;
    float* logits = malloc(nl * 4);
    float* q = malloc(nq * 4);
    int32_t* xg = malloc((size_t)B * G * 4);
    int32_t* xs = malloc((size_t)B * G * 4);
    float* coins = malloc((size_t)B * R * 4);
    float* temp = malloc((size_t)B * 4);
    if (!logits || !q || !xg || !xs || !coins || !temp) return 1;
    if (!read_all(fi, logits, nl * 4) || !read_all(fi, q, nq * 4) ||
        !read_all(fi, xg, (size_t)B * G * 4) || !read_all(fi, xs, (size_t)B * G * 4) ||
        !read_all(fi, coins, (size_t)B * R * 4) || !read_all(fi, temp, (size_t)B * 4))
        return 1;
    fclose(fi);

    void *d_logits, *d_q, *d_xg, *d_xs, *d_coins, *d_temp, *d_accg, *d_outg, *d_accc, *d_outc,
        *d_probs, *d_wsg, *d_wsc;
    const size_t wsg = spec_workspace_bytes(SPEC_OP_GREEDY, B, R, V);
    const size_t wsc = spec_workspace_bytes(SPEC_OP_CHAIN, B, R, V);
    if (wsg == 0 || wsc == 0) return 3;
    HIP(hipMalloc(&d_logits, nl * 4));
    HIP(hipMalloc(&d_q, nq * 4));
    HIP(hipMalloc(&d_xg, (size_t)B * G * 4));
    HIP(hipMalloc(&d_xs, (size_t)B * G * 4));
    HIP(hipMalloc(&d_coins, (size_t)B * R * 4));
    HIP(hipMalloc(&d_temp, (size_t)B * 4));
    HIP(hipMalloc(&d_accg, (size_t)B * 4));
    HIP(hipMalloc(&d_outg, (size_t)B * R * 4));
    HIP(hipMalloc(&d_accc, (size_t)B * 4));
    HIP(hipMalloc(&d_outc, (size_t)B * R * 4));
    HIP(hipMalloc(&d_probs, (size_t)B * R * 4));
    HIP(hipMalloc(&d_wsg, wsg));  /* hipMalloc returns 256-byte aligned memory */
    HIP(hipMalloc(&d_wsc, wsc));
    HIP(hipMemset(d_wsg, 0, wsg));  /* zero once, before the first call */
    HIP(hipMemset(d_wsc, 0, wsc));
    HIP(hipMemcpy(d_logits, logits, nl * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_q, q, nq * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_xg, xg, (size_t)B * G * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_xs, xs, (size_t)B * G * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_coins, coins, (size_t)B * R * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_temp, temp, (size_t)B * 4, hipMemcpyHostToDevice));

    int rc = spec_verify_greedy(d_logits, SPEC_F32, d_xg, B, G, V, d_accg, d_outg, d_wsg, wsg,
                                NULL);
    if (rc != SPEC_OK) {
        fprintf(stderr, "spec_verify_greedy: %s\n", spec_status_str(rc));
        return 3;
    }
    rc = spec_verify_chain(d_logits, SPEC_F32, d_q, d_xs, d_coins, d_temp, B, G, V, d_accc,
                           d_outc, d_probs, d_wsc, wsc, NULL);
    if (rc != SPEC_OK) {
        fprintf(stderr, "spec_verify_chain: %s\n", spec_status_str(rc));
        return 3;
    }
    HIP(hipDeviceSynchronize());

    int32_t* accg = malloc((size_t)B * 4);
    int32_t* outg = malloc((size_t)B * R * 4);
    int32_t* accc = malloc((size_t)B * 4);
    int32_t* outc = malloc((size_t)B * R * 4);
    float* probs = malloc((size_t)B * R * 4);
    if (!accg || !outg || !accc || !outc || !probs) return 1;
    HIP(hipMemcpy(accg, d_accg, (size_t)B * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(outg, d_outg, (size_t)B * R * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(accc, d_accc, (size_t)B * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(outc, d_outc, (size_t)B * R * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(probs, d_probs, (size_t)B * R * 4, hipMemcpyDeviceToHost));
    FILE* fo = fopen(argv[2], "wb");
    if (!fo) return 1;
    fwrite(accg, 4, (size_t)B, fo);
    fwrite(outg, 4, (size_t)B * R, fo);
    fwrite(accc, 4, (size_t)B, fo);
    fwrite(outc, 4, (size_t)B * R, fo);
    fwrite(probs, 4, (size_t)B * R, fo);
    fclose(fo);
    void* bufs[13] = {d_logits, d_q, d_xg, d_xs, d_coins, d_temp, d_accg, d_outg, d_accc, d_outc,
                      d_probs, d_wsg, d_wsc};
    for (int i = 0; i < 13; ++i) HIP(hipFree(bufs[i]));
    free(logits); free(q); free(xg); free(xs); free(coins); free(temp);
    free(accg); free(outg); free(accc); free(outc); free(probs);
    return 0;
}
