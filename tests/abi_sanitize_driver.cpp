// Host-only driver for the C ABI's validation and workspace arithmetic, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host side (the
// device code is untouched). Every compute entry point is called only with
// arguments that validation rejects, so no kernel is ever launched; the
// workspace queries run over a sweep of shapes up to the largest the ABI takes.
// Prints one line per failure and exits non-zero if any check failed.
#include <cstdint>
#include <cstdio>
#include <limits>

#include "msa.h"

static int g_fail = 0;
static int g_checks = 0;

#define EXPECT_EQ(got, want)                                                                          \
    do {                                                                                              \
        ++g_checks;                                                                                   \
        const int got_ = (int)(got), want_ = (int)(want);                                             \
        if (got_ != want_) {                                                                          \
            std::printf("FAIL line %d: %s -> %d, expected %d\n", __LINE__, #got, got_, want_);         \
            ++g_fail;                                                                                 \
        }                                                                                             \
    } while (0)

static msa_shape make(int B, int N, int hq, int hkv, int k) {
    msa_shape s;
    s.batch = B;
    s.seqlen = N;
    s.h_q = hq;
    s.h_kv = hkv;
    s.h_idx = hkv;
    s.head_dim = 128;
    s.idx_dim = 128;
    s.block_size = 128;
    s.top_k = k;
    s.softmax_scale = 0.08838834764831845f;
    s.flags = MSA_CAUSAL;
    return s;
}

// A non-null address that is never dereferenced on the host: every call below is
// rejected by validation before any launch.
static void* const P = reinterpret_cast<void*>(static_cast<uintptr_t>(0x1000));
static float* const PF = reinterpret_cast<float*>(static_cast<uintptr_t>(0x1000));
static int32_t* const PI = reinterpret_cast<int32_t*>(static_cast<uintptr_t>(0x1000));
static hipStream_t const S = nullptr;

static void sweep_workspace_sizes() {
    const int Bs[] = {1, 2, 3, 255, 65535, 65536, 1 << 20, std::numeric_limits<int32_t>::max(), 0, -1};
    const int Ns[] = {128, 1024, 8192, 131072, 1 << 20, (1 << 23) - 128, 1 << 23, 200,
                      std::numeric_limits<int32_t>::max(), 0, -128};
    const int heads[][2] = {{4, 1}, {64, 4}, {32, 8}, {128, 1}, {256, 1}, {6, 3}, {65536, 1}, {1, 0}};
    const int ks[] = {1, 4, 16, 17, 18, 65, 66, 256, 257, std::numeric_limits<int32_t>::max(), 0, -5};
    for (int B : Bs)
        for (int N : Ns)
            for (auto& h : heads)
                for (int k : ks)
                    for (int op = MSA_OP_INDEX_SCORES; op <= MSA_OP_INDEX_BWD; ++op) {
                        msa_shape s = make(B, N, h[0], h[1], k);
                        size_t bytes = 7;
                        const msa_status st = msa_workspace_size(&s, (msa_op)op, &bytes);
                        ++g_checks;
                        if (st != MSA_OK && bytes != 7) {
                            std::printf("FAIL: rejected shape wrote the size (B=%d N=%d op=%d)\n", B, N, op);
                            ++g_fail;
                        }
                        if (st == MSA_OK && op == MSA_OP_SPARSE_ATTN_FWD && bytes == 0) {
                            std::printf("FAIL: zero forward workspace (B=%d N=%d)\n", B, N);
                            ++g_fail;
                        }
                    }
}

int main() {
    msa_shape ok = make(1, 1024, 4, 1, 4);
    size_t bytes = 0;

    // workspace query
    EXPECT_EQ(msa_workspace_size(nullptr, MSA_OP_FWD, &bytes), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_workspace_size(&ok, MSA_OP_FWD, nullptr), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_workspace_size(&ok, (msa_op)99, &bytes), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_workspace_size(&ok, (msa_op)-1, &bytes), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_workspace_size(&ok, MSA_OP_FWD, &bytes), MSA_OK);
    const size_t fwd_ws = bytes;

    // shape checks
    msa_shape s = ok;
    s.flags = 0;
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = ok;
    s.softmax_scale = std::numeric_limits<float>::quiet_NaN();
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_INVALID_ARG);
    s = ok;
    s.softmax_scale = std::numeric_limits<float>::infinity();
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_INVALID_ARG);
    s = ok;
    s.h_kv = 0;
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_INVALID_ARG);
    s = ok;
    s.h_q = std::numeric_limits<int32_t>::min();
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_INVALID_ARG);
    s = ok;
    s.head_dim = 64;
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = ok;
    s.h_idx = 2;
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = make(1, 1024, 12, 4, 4);  // G = 3
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = make(1, 1 << 23, 4, 1, 4);
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = make(std::numeric_limits<int32_t>::max(), (1 << 23) - 128, 128, 1, 256);
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = make(1, 4096, 4, 1, 257);
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_FWD, &bytes), MSA_ERR_UNSUPPORTED);
    s = make(1, 1 << 21, 4, 1, 65);  // decode capacity at its limit
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_DECODE, &bytes), MSA_OK);
    s = make(1, (1 << 21) + 128, 4, 1, 65);
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_DECODE, &bytes), MSA_ERR_UNSUPPORTED);
    s = make(1, 4096, 4, 1, 66);
    EXPECT_EQ(msa_workspace_size(&s, MSA_OP_DECODE, &bytes), MSA_ERR_UNSUPPORTED);
    sweep_workspace_sizes();

    // compute entry points: null pointers and bad shapes are rejected before any launch
    msa_shape bad = ok;
    bad.seqlen = 200;
    EXPECT_EQ(msa_index_scores(nullptr, P, P, PF, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_index_scores(&ok, nullptr, P, PF, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_index_scores(&ok, P, P, nullptr, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_index_scores(&bad, P, P, PF, S), MSA_ERR_UNSUPPORTED);
    EXPECT_EQ(msa_block_topk(&ok, nullptr, PI, nullptr, 0, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_block_topk(&bad, PF, PI, nullptr, 0, S), MSA_ERR_UNSUPPORTED);
    msa_shape long_rows = make(1, 1 << 20, 4, 1, 16);  // 8192 blocks: past the selection kernel's list
    EXPECT_EQ(msa_block_topk(&long_rows, PF, PI, nullptr, 0, S), MSA_ERR_UNSUPPORTED);
    EXPECT_EQ(msa_index_topk(&ok, P, nullptr, PI, nullptr, 0, S), MSA_ERR_INVALID_ARG);
    msa_shape k18 = make(1, 4096, 4, 1, 18);  // two-kernel selection: needs the pooled workspace
    EXPECT_EQ(msa_index_topk(&k18, P, P, PI, nullptr, 0, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_index_topk(&k18, P, P, PI, P, 16, S), MSA_ERR_WORKSPACE);

    EXPECT_EQ(msa_sparse_attn_fwd(&ok, P, P, nullptr, PI, P, PF, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_fwd(&ok, P, P, P, PI, P, PF, nullptr, fwd_ws, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_sparse_attn_fwd(&ok, P, P, P, PI, P, PF, P, 1000, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_sparse_attn_plan(&ok, nullptr, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_plan(&ok, PI, P, fwd_ws - 1, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_sparse_attn_partial(&ok, P, nullptr, P, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_partial(&ok, P, P, P, nullptr, fwd_ws, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_sparse_attn_combine(&ok, P, P, P, PI, nullptr, PF, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_combine(&ok, nullptr, P, P, PI, P, PF, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_combine(&ok, P, P, nullptr, PI, P, PF, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_combine(&ok, P, P, P, PI, P, PF, P, 0, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_fwd(&ok, P, P, P, P, P, PI, P, nullptr, P, fwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_fwd(&ok, P, P, P, P, P, PI, P, PF, nullptr, 0, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_fwd(&ok, P, P, P, P, P, PI, P, PF, P, 255, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_fwd(&bad, P, P, P, P, P, PI, P, PF, P, fwd_ws, S), MSA_ERR_UNSUPPORTED);

    EXPECT_EQ(msa_workspace_size(&ok, MSA_OP_SPARSE_ATTN_BWD, &bytes), MSA_OK);
    const size_t bwd_ws = bytes;
    EXPECT_EQ(msa_sparse_attn_bwd(&ok, P, P, P, P, PF, nullptr, PI, P, P, P, P, bwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_sparse_attn_bwd(&ok, P, P, P, P, PF, P, PI, P, P, P, P, bwd_ws - 1, S), MSA_ERR_WORKSPACE);
    msa_shape huge = make(4, 1 << 22, 128, 1, 1);  // 2^31 query rows: past the backward's 32-bit rows
    EXPECT_EQ(msa_sparse_attn_bwd(&huge, P, P, P, P, PF, P, PI, P, P, P, P, ~(size_t)0, S), MSA_ERR_UNSUPPORTED);

    EXPECT_EQ(msa_workspace_size(&ok, MSA_OP_INDEX_BWD, &bytes), MSA_OK);
    const size_t ibwd_ws = bytes;
    EXPECT_EQ(msa_index_bwd(&ok, P, P, P, P, PF, PI, 0.1f, 1.0f, P, nullptr, P, ibwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_index_bwd(&ok, P, P, P, P, PF, PI, 0.0f, 1.0f, P, P, P, ibwd_ws, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_index_bwd(&ok, P, P, P, P, PF, PI, 0.1f, std::numeric_limits<float>::quiet_NaN(), P, P, P, ibwd_ws,
                            S),
              MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_index_bwd(&ok, P, P, P, P, PF, PI, 0.1f, 1.0f, P, P, P, ibwd_ws - 1, S), MSA_ERR_WORKSPACE);
    msa_shape g64 = make(1, 1024, 64, 1, 4);
    EXPECT_EQ(msa_index_bwd(&g64, P, P, P, P, PF, PI, 0.1f, 1.0f, P, P, P, ~(size_t)0, S), MSA_ERR_UNSUPPORTED);

    msa_shape dec = make(3, 4096, 8, 2, 4);
    EXPECT_EQ(msa_workspace_size(&dec, MSA_OP_DECODE, &bytes), MSA_OK);
    const size_t dec_ws = bytes;
    EXPECT_EQ(msa_decode_index_scores(&dec, P, P, nullptr, PF, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_decode_topk(&dec, PF, PI, nullptr, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_decode_attn(&dec, P, P, P, PI, PI, nullptr, PF, nullptr, 0, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_decode_attn(&dec, P, P, P, PI, PI, P, PF, P, 16, S), MSA_ERR_WORKSPACE);  // split records
    EXPECT_EQ(msa_decode(&dec, P, P, P, P, P, PI, PI, P, PF, nullptr, dec_ws, S), MSA_ERR_WORKSPACE);
    EXPECT_EQ(msa_decode(&dec, P, P, P, P, P, PI, PI, P, PF, P, dec_ws - 1, S), MSA_ERR_WORKSPACE);
    msa_shape dec_bad = dec;
    dec_bad.seqlen = 4000;
    EXPECT_EQ(msa_decode(&dec_bad, P, P, P, P, P, PI, PI, P, PF, P, dec_ws, S), MSA_ERR_UNSUPPORTED);

    // the allocation-free decode: rejected before it looks anything up on a device
    EXPECT_EQ(msa_decode_noalloc(&dec, P, P, P, P, P, PI, PI, P, nullptr, S), MSA_ERR_INVALID_ARG);
    EXPECT_EQ(msa_decode_noalloc(&dec_bad, P, P, P, P, P, PI, PI, P, PF, S), MSA_ERR_UNSUPPORTED);
    msa_shape dec_big = make(128, 1 << 21, 8, 8, 16);  // 128 * 8 * 16384 * 4 B = 64 MiB of pooled scores
    EXPECT_EQ(msa_decode_noalloc(&dec_big, P, P, P, P, P, PI, PI, P, PF, S), MSA_ERR_WORKSPACE);

    // status strings: never NULL, also for values outside the enum
    for (int st = -3; st <= 8; ++st) {
        ++g_checks;
        if (msa_status_string((msa_status)st) == nullptr) {
            std::printf("FAIL: NULL status string for %d\n", st);
            ++g_fail;
        }
    }

    std::printf("%d checks, %d failures\n", g_checks, g_fail);
    return g_fail == 0 ? 0 : 1;
}
