// abi_driver.cpp -- exercises the host side of the verify library's C ABI with arguments
// that every entry point must reject before it touches the device: NULL pointers, sizes
// outside the supported ranges, unknown dtypes and modes, misaligned or short workspaces,
// bad launch options, and the static-scratch entry point's size limit.  Built with the
// address and undefined-behaviour sanitizers on the host pass only (tests/test_sanitizers.py);
// no GPU is needed, since no call gets as far as a launch.  Exit status 0 when every call
// returned the expected status.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spec_verify.h"

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                            \
        }                                                                        \
    } while (0)

int main() {
    void* P = reinterpret_cast<void*>(uintptr_t(1) << 20);  // never dereferenced
    const float* Pf = static_cast<const float*>(P);
    const int32_t* Pi = static_cast<const int32_t*>(P);
    int32_t* Po = static_cast<int32_t*>(P);
    const size_t wsc = spec_workspace_bytes(SPEC_OP_CHAIN, 3, 5, 2000);
    const size_t wsg = spec_workspace_bytes(SPEC_OP_GREEDY, 3, 5, 2000);
    const size_t wst = spec_workspace_bytes(SPEC_OP_TREE, 3, 16, 2000);
    const size_t wsm = spec_workspace_bytes(SPEC_OP_TREE_MSS, 3, 16, 2000);
    const size_t wsf = spec_workspace_bytes(SPEC_OP_CHAIN_FILTERED, 3, 5, 2000);
    CHECK(wsc > 0 && wsg > 0 && wst > 0 && wsm > 0 && wsf > 0);
    CHECK(spec_workspace_bytes(SPEC_OP_CHAIN, 3, 66, 10) == 0);
    CHECK(spec_workspace_bytes(SPEC_OP_TREE, 3, 1025, 10) == 0);
    CHECK(spec_workspace_bytes(9, 3, 5, 10) == 0);
    CHECK(spec_workspace_bytes(SPEC_OP_CHAIN, -1, 5, 10) == 0);
    for (int s = 1; s >= -8; --s) CHECK(spec_status_str(s) != nullptr && std::strlen(spec_status_str(s)) > 0);

    // greedy
    CHECK(spec_verify_greedy(nullptr, SPEC_BF16, Pi, 3, 4, 2000, Po, Po, P, wsg, nullptr) == SPEC_ERR_NULL);
    CHECK(spec_verify_greedy(P, 7, Pi, 3, 4, 2000, Po, Po, P, wsg, nullptr) == SPEC_ERR_DTYPE);
    CHECK(spec_verify_greedy(P, SPEC_BF16, Pi, 3, 65, 2000, Po, Po, P, wsg, nullptr) == SPEC_ERR_SHAPE);
    CHECK(spec_verify_greedy(P, SPEC_BF16, Pi, 3, 4, 2000, Po, Po, P, 64, nullptr) == SPEC_ERR_WORKSPACE);
    CHECK(spec_verify_greedy(static_cast<char*>(P) + 1, SPEC_BF16, Pi, 3, 4, 2000, Po, Po, P, wsg,
                             nullptr) == SPEC_ERR_PARAM);
    CHECK(spec_verify_greedy(P, SPEC_BF16, Pi, 0, 4, 2000, Po, Po, P, wsg, nullptr) == SPEC_OK);
    // chain
    CHECK(spec_verify_chain(P, SPEC_BF16, nullptr, Pi, Pf, Pf, 3, 4, 2000, Po, Po, nullptr, P, wsc,
                            nullptr) == SPEC_ERR_NULL);
    CHECK(spec_verify_chain(P, SPEC_BF16, Pf, Pi, Pf, Pf, 3, 0, 2000, Po, Po, nullptr, P, wsc,
                            nullptr) == SPEC_ERR_SHAPE);
    CHECK(spec_verify_chain(P, SPEC_BF16, Pf, Pi, Pf, Pf, 3, 4, 2000, Po, Po, nullptr,
                            static_cast<char*>(P) + 16, wsc, nullptr) == SPEC_ERR_WORKSPACE);
    spec_options bad;
    std::memset(&bad, 0, sizeof bad);
    bad.path = 5;
    CHECK(spec_verify_chain_opt(P, SPEC_BF16, Pf, Pi, Pf, Pf, 3, 4, 2000, Po, Po, nullptr, P, wsc,
                                nullptr, &bad) == SPEC_ERR_PARAM);
    bad.path = 0;
    bad.spin_limit = -3;
    CHECK(spec_verify_greedy_opt(P, SPEC_BF16, Pi, 3, 4, 2000, Po, Po, P, wsg, nullptr, &bad) ==
          SPEC_ERR_PARAM);
    CHECK(spec_verify_chain_noalloc(P, SPEC_BF16, Pf, Pi, Pf, Pf, 4096, 4, 152064, Po, Po, nullptr,
                                    nullptr) == SPEC_ERR_TOO_LARGE);
    CHECK(spec_verify_chain_noalloc(P, SPEC_BF16, Pf, Pi, Pf, Pf, 0, 4, 2000, Po, Po, nullptr,
                                    nullptr) == SPEC_OK);
    // tree
    CHECK(spec_verify_tree(P, SPEC_F32, Pi, Pi, Pf, Pf, 3, 16, 2000, 4, 3, 1.f, 1.f, Po, Po, Po,
                           nullptr, P, wst, nullptr) == SPEC_ERR_PARAM);
    CHECK(spec_verify_tree(P, SPEC_F32, Pi, Pi, Pf, Pf, 3, 1025, 2000, 4, 1, 1.f, 1.f, Po, Po, Po,
                           nullptr, P, wst, nullptr) == SPEC_ERR_SHAPE);
    CHECK(spec_verify_tree(P, SPEC_F32, Pi, Pi, nullptr, Pf, 3, 16, 2000, 4, 1, 1.f, 1.f, Po, Po, Po,
                           nullptr, P, wst, nullptr) == SPEC_ERR_NULL);
    CHECK(spec_verify_tree_opt(P, SPEC_F32, Pi, Pi, Pf, Pf, 3, 16, 2000, 4, 1, 0.f, 1.f, Po, Po, Po,
                               nullptr, P, wst, nullptr, nullptr) == SPEC_ERR_PARAM);
    CHECK(spec_verify_tree_mss(P, SPEC_F32, Pf, Pi, Pi, Pf, Pf, 3, 16, 2000, 0, Po, Po, Po, nullptr,
                               P, wsm, nullptr) == SPEC_ERR_SHAPE);
    CHECK(spec_verify_tree_mss_opt(P, SPEC_F32, Pf, Pi, Pi, Pf, Pf, 3, 16, 2000, 4, Po, Po, Po,
                                   nullptr, P, wsm - 1, nullptr, nullptr) == SPEC_ERR_WORKSPACE);
    CHECK(spec_verify_chain_filtered(P, nullptr, SPEC_BF16, Pi, Pf, Pf, nullptr, nullptr, 3, 4, 2000,
                                     Po, Po, nullptr, P, wsf, nullptr) == SPEC_ERR_NULL);
    CHECK(spec_tree_mask(Pi, nullptr, 3, 0, static_cast<uint32_t*>(P), Po, nullptr) == SPEC_ERR_SHAPE);
    CHECK(spec_tree_commit_kv(Pi, Pi, 3, 4, 8, P, P, 0, Po, nullptr) == SPEC_ERR_SHAPE);
    CHECK(spec_calib_exp(0, 1, static_cast<float*>(P), nullptr) == SPEC_ERR_PARAM);
    CHECK(spec_calib_read(P, 24, static_cast<float*>(P), nullptr) == SPEC_ERR_PARAM);
    std::printf("ABI driver: all argument checks passed\n");
    return 0;
}
