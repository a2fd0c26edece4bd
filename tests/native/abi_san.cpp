// Host program for the sanitizer tier: drives the library's host-side code
// (shape rules, packed sizes, the route planners of every kernel, workspace
// sizes, stream sizes, status strings) over many seeded shapes, and every
// entry point with arguments that its validation rejects before any device
// call -- so that AddressSanitizer and UndefinedBehaviorSanitizer watch the
// planners' integer arithmetic and the validation paths.  It makes no GPU
// call.  Prints "ok <calls>" and exits 0 when every call behaved.
#include <cstdint>
#include <cstdio>

#include "ctconv.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static int64_t rnd(int64_t lo, int64_t hi) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return lo + (int64_t)(st % (uint64_t)(hi - lo + 1));
}

#define EXPECT(cond)                                              \
    do {                                                          \
        if (!(cond)) {                                            \
            std::printf("failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                             \
        }                                                         \
    } while (0)

int main() {
    long calls = 0;
    EXPECT(ctconv_abi_version() > 0);
    for (int s = 0; s <= CTCONV_ERR_SCRATCH; ++s)
        EXPECT(ctconv_status_string((ctconv_status)s) != nullptr);

    // planners over seeded shapes, valid and invalid
    for (int it = 0; it < 20000; ++it) {
        const int nd = 1 + (int)rnd(0, 1);
        int64_t in[2], k[2], s[2], p[2], op[2], d[2], out[2];
        for (int a = 0; a < nd; ++a) {
            in[a] = rnd(0, 3) == 0 ? rnd(-2, 3) : rnd(1, 5000);
            k[a] = rnd(0, 9) == 0 ? rnd(-1, 1) : rnd(1, 64);
            s[a] = rnd(0, 9) == 0 ? rnd(-1, 0) : rnd(1, 16);
            d[a] = rnd(0, 3) == 0 ? rnd(1, 7) : 1;
            p[a] = rnd(0, 9) == 0 ? rnd(-2, 100) : rnd(0, k[a] > 0 ? k[a] : 1);
            op[a] = rnd(0, 4) == 0 ? rnd(-1, 8) : 0;
        }
        const int64_t N = rnd(0, 9) == 0 ? rnd(-1, 0) : rnd(1, 16);
        const int64_t Ci = rnd(0, 19) == 0 ? rnd(-1, 0) : rnd(1, 5000);
        const int64_t Co = rnd(0, 19) == 0 ? rnd(-1, 0) : rnd(1, 600);
        // (valid enum values only: out-of-range ones, which a C caller may
        // pass, are covered by the host tests through ctypes)
        const ctconv_dtype dt = (ctconv_dtype)rnd(0, 2);
        ctconv_output_shape(nd, in, k, s, p, op, d, out);
        size_t pb = 0, wb = 0;
        ctconv_packed_bytes(nd, Ci, Co, k, s, dt, &pb);
        ctconv_route r;
        ctconv_query_route(N, Ci, Co, nd, in, k, s, p, op, d, dt, &r);
        ctconv_workspace_bytes(N, Ci, Co, nd, in, k, s, p, op, d, dt, &wb);
        ctconv_dw_kernel dk;
        const int64_t M = rnd(1, 3);
        ctconv_depthwise_query_kernel(N, Ci, Ci * M, nd, in, k, s, p, op, d, dt, &dk);
        int64_t yl, tl, wsb;
        ctconv_stream_sizes(N, Co, rnd(-1, 40), k[0], s[0], dt, &yl, &tl, &wsb);
        calls += 6;
    }

    // validation: rejected before any device call
    const int64_t in1[1] = {100}, k1[1] = {8}, s1[1] = {4}, p1[1] = {2}, op1[1] = {0},
                  d1[1] = {1};
    char* base = reinterpret_cast<char*>(0x100000);  // never dereferenced
    void* x = base;
    void* w = base + 0x10000;
    void* y = base + 0x20000;
    EXPECT(ctconv_forward(nullptr, w, nullptr, y, 2, 16, 8, 1, in1, k1, s1, p1, op1, d1,
                          CTCONV_BF16, nullptr) == CTCONV_ERR_NULL);
    EXPECT(ctconv_forward(base + 1, w, nullptr, y, 2, 16, 8, 1, in1, k1, s1, p1, op1, d1,
                          CTCONV_BF16, nullptr) == CTCONV_ERR_ALIGN);
    EXPECT(ctconv_forward(x, w, nullptr, y, 2, 0, 8, 1, in1, k1, s1, p1, op1, d1, CTCONV_BF16,
                          nullptr) == CTCONV_ERR_SHAPE);
    EXPECT(ctconv_forward(x, w, nullptr, y, 2, 16, 8, 3, in1, k1, s1, p1, op1, d1, CTCONV_BF16,
                          nullptr) == CTCONV_ERR_PARAM);
    const int64_t s0[1] = {0};
    EXPECT(ctconv_forward_route(x, w, nullptr, y, 2, 16, 8, 1, in1, k1, s0, p1, op1, d1,
                                CTCONV_BF16, CTCONV_ROUTE_GATHER, nullptr) == CTCONV_ERR_PARAM);
    EXPECT(ctconv_forward_act(x, w, nullptr, nullptr, 2, 16, 8, 1, in1, k1, s1, p1, op1, d1,
                              CTCONV_BF16, CTCONV_ACT_ELU, CTCONV_ROUTE_AUTO,
                              nullptr) == CTCONV_ERR_NULL);
    // the iSTFT shape splits its reduction: a short workspace is rejected
    const int64_t inI[1] = {345}, kI[1] = {4096}, sI[1] = {1024}, pI[1] = {0};
    size_t need = 0;
    EXPECT(ctconv_workspace_bytes(8, 4098, 1, 1, inI, kI, sI, pI, op1, d1, CTCONV_F32, &need) ==
           CTCONV_OK);
    EXPECT(need > 0);
    EXPECT(ctconv_forward_ws(x, w, nullptr, y, 8, 4098, 1, 1, inI, kI, sI, pI, op1, d1,
                             CTCONV_F32, CTCONV_ACT_NONE, base + 0x30000, need - 16,
                             nullptr) == CTCONV_ERR_WORKSPACE);
    // more than the no-allocation scratch: rejected before any device call
    const int64_t inB[1] = {345 * 6};
    EXPECT(ctconv_workspace_bytes(64, 4098, 1, 1, inB, kI, sI, pI, op1, d1, CTCONV_F32, &need) ==
           CTCONV_OK);
    if (need > ctconv_scratch_bytes())
        EXPECT(ctconv_forward_noalloc(x, w, nullptr, y, 64, 4098, 1, 1, inB, kI, sI, pI, op1, d1,
                                      CTCONV_F32, CTCONV_ACT_NONE,
                                      nullptr) == CTCONV_ERR_SCRATCH);
    EXPECT(ctconv_prepack(nullptr, w, 1, 16, 8, k1, s1, CTCONV_BF16, nullptr) == CTCONV_ERR_NULL);
    EXPECT(ctconv_elu(nullptr, y, 16, CTCONV_BF16, nullptr) == CTCONV_ERR_NULL);
    EXPECT(ctconv_istft_normalize(x, w, y, 2, 10, 6, 5, CTCONV_F32, nullptr) == CTCONV_ERR_SHAPE);
    EXPECT(ctconv_stream_step(x, w, nullptr, y, nullptr, nullptr, base + 0x30000, 1, 16, 8, 4, 2,
                              4, CTCONV_BF16, CTCONV_ACT_NONE, nullptr) == CTCONV_ERR_PARAM);
    EXPECT(ctconv_depthwise_forward(nullptr, w, nullptr, y, 2, 16, 16, 1, in1, k1, s1, p1, op1,
                                    d1, CTCONV_BF16, CTCONV_ACT_NONE,
                                    nullptr) == CTCONV_ERR_NULL);
    calls += 16;
    std::printf("ok %ld\n", calls);
    return 0;
}
