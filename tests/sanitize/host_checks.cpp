// Memory- and UB-safety driver for the host side of libnsa_sel (test
// infrastructure): the library's sources are compiled for the host only,
// with AddressSanitizer and UndefinedBehaviorSanitizer, together with this
// driver, which calls every entry point with arguments each host check must
// reject -- null pointers, bad and huge sizes, misaligned and overlapping
// buffers, short workspaces -- and the size queries over a sweep of shapes.
// Every call here returns before any HIP call, so no GPU is needed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nsa_dense.h"
#include "nsa_sel.h"
#include "nsa_sel_bwd.h"
#include "nsa_topk.h"

static int failures = 0;
static void expect(bool ok, const char *what, int got) {
    if (!ok) {
        fprintf(stderr, "FAILED: %s (status %d)\n", what, got);
        failures++;
    }
}

static void *A(int i) { return (void *)((uintptr_t)(i + 1) << 36); }  // distinct aligned fake addresses

int main() {
    // nsa_sel_fwd and its variants
    typedef int (*Fwd)(const void *, const void *, const void *, const int32_t *, void *, float *, int, int, int, int,
                       int, int, int, int, hipStream_t);
    const Fwd fwds[3] = {nsa_sel_fwd, nsa_sel_fwd_bf16, nsa_sel_fwd_unpipelined};
    for (Fwd f : fwds) {
        const int32_t *I = (const int32_t *)A(3);
        float *L = (float *)A(5);
        int rc;
        rc = f(nullptr, A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_NULL, "fwd null", rc);
        const int shapes[][8] = {{0, 64, 64, 8, 2, 64, 32, 4}, {1, -5, 64, 8, 2, 64, 32, 4},
                                 {1, 64, 64, 8, 3, 64, 32, 4}, {1, 64, 64, 8, 2, 64, 32, 0},
                                 {1, 64, 64, 8, 2, 64, 0, 4}};
        for (const auto &s : shapes) {
            rc = f(A(0), A(1), A(2), I, A(4), L, s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], 0);
            expect(rc == NSA_SEL_ERR_SHAPE, "fwd shape", rc);
        }
        rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 96, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_UNSUPPORTED, "fwd D", rc);
        rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 64, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_UNSUPPORTED, "fwd gs", rc);
        rc = f(A(0), A(1), A(2), I, A(4), L, 1 << 12, 1 << 20, 64, 1, 1, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_RANGE, "fwd range", rc);
        rc = f(A(0), A(1), (char *)A(2) + 8, I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_ALIGN, "fwd align", rc);
        rc = f(A(0), A(1), A(2), I, (char *)A(0) + 64, L, 1, 64, 64, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_ALIAS, "fwd alias", rc);
        rc = f(A(0), A(1), A(2), I, A(4), (float *)A(4), 1, 64, 64, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_ALIAS, "fwd alias outputs", rc);
    }
    // the workspace forward: size sweep, then rejected calls
    {
        size_t n = 0, prev = 0;
        for (int M = 32; M <= 1 << 17; M *= 2) {
            int rc = nsa_sel_fwd_workspace_size(1, M, M, 64, 8, 128, 64, 16, &n);
            expect(rc == NSA_SEL_OK && n >= prev && n % 4 == 0, "fwd workspace grows", rc);
            prev = n;
            rc = nsa_sel_fwd_workspace_size(2, M, M + 17, 48, 4, 64, 32, 70, &n);
            expect(rc == NSA_SEL_OK && n > 0, "fwd workspace ragged", rc);
        }
        int rc = nsa_sel_fwd_workspace_size(1, 64, 64, 8, 2, 64, 32, 4, nullptr);
        expect(rc == NSA_SEL_ERR_NULL, "fwd workspace null", rc);
        rc = nsa_sel_fwd_workspace_size(1, 64, 64, 8, 3, 64, 32, 4, &n);
        expect(rc == NSA_SEL_ERR_SHAPE, "fwd workspace shape", rc);
        const int32_t *I = (const int32_t *)A(3);
        float *L = (float *)A(5);
        size_t need = 0;
        nsa_sel_fwd_workspace_size(1, 64, 64, 8, 2, 64, 32, 4, &need);
        typedef int (*FwdWs)(const void *, const void *, const void *, const int32_t *, void *, float *, int, int,
                             int, int, int, int, int, int, void *, size_t, hipStream_t);
        const FwdWs fws[2] = {nsa_sel_fwd_ws, nsa_sel_fwd_bf16_ws};
        for (FwdWs f : fws) {
            rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, nullptr, need, 0);
            expect(rc == NSA_SEL_ERR_WORKSPACE, "fwd_ws null workspace", rc);
            rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, A(6), need - 1, 0);
            expect(rc == NSA_SEL_ERR_WORKSPACE, "fwd_ws short workspace", rc);
            rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, (char *)A(6) + 16, need, 0);
            expect(rc == NSA_SEL_ERR_WORKSPACE, "fwd_ws misaligned workspace", rc);
            rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, A(1), need, 0);
            expect(rc == NSA_SEL_ERR_ALIAS, "fwd_ws workspace over K", rc);
            rc = f(nullptr, A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 64, 32, 4, A(6), need, 0);
            expect(rc == NSA_SEL_ERR_NULL, "fwd_ws null", rc);
            rc = f(A(0), A(1), A(2), I, A(4), L, 1, 64, 64, 8, 2, 96, 32, 4, A(6), need, 0);
            expect(rc == NSA_SEL_ERR_UNSUPPORTED, "fwd_ws D", rc);
        }
    }
    // dense and window
    {
        int rc = nsa_dense_fwd(A(0), A(1), nullptr, A(4), (float *)A(5), 1, 64, 64, 8, 2, 64, 0);
        expect(rc == NSA_SEL_ERR_NULL, "dense null", rc);
        rc = nsa_dense_fwd(A(0), A(1), A(2), A(4), (float *)A(5), 1, 64, 64, 8, 2, 80, 0);
        expect(rc != NSA_SEL_OK, "dense D", rc);
        rc = nsa_window_fwd(A(0), A(1), A(2), A(0), (float *)A(5), 1, 64, 64, 8, 2, 64, 8, 0, 0);
        expect(rc == NSA_SEL_ERR_ALIAS, "window alias", rc);
        rc = nsa_window_fwd_bf16(A(0), A(1), A(2), A(4), (float *)A(5), 1, 0, 64, 8, 2, 64, 8, 0, 0);
        expect(rc == NSA_SEL_ERR_SHAPE, "window shape", rc);
    }
    // backward: workspace sizes over a sweep, then rejected calls
    {
        size_t n = 0, prev = 0;
        for (int M = 32; M <= 1 << 17; M *= 2) {
            int rc = nsa_sel_bwd_workspace_size(1, M, M, 64, 8, 128, 64, 16, &n);
            expect(rc == NSA_SEL_OK && n > prev && n % 256 == 0, "bwd workspace grows", rc);
            prev = n;
            rc = nsa_sel_bwd_workspace_size(2, M, M + 17, 48, 4, 64, 32, 40, &n);
            expect(rc == NSA_SEL_OK, "bwd workspace ragged", rc);
        }
        int rc = nsa_sel_bwd_workspace_size(1, 64, 64, 8, 2, 64, 32, 4, nullptr);
        expect(rc == NSA_SEL_ERR_NULL, "bwd workspace null", rc);
        rc = nsa_sel_bwd_workspace_size(1, 1 << 20, 1024, 16, 1, 128, 64, 4, &n);
        expect(rc == NSA_SEL_ERR_RANGE, "bwd workspace range", rc);
        nsa_sel_bwd_workspace_size(1, 256, 256, 8, 2, 64, 32, 4, &n);
        const void *in[7] = {A(0), A(1), A(2), A(3), A(4), A(5), A(6)};
        rc = nsa_sel_bwd(in[0], in[1], in[2], (const int32_t *)in[3], in[4], (const float *)in[5], in[6],
                         (float *)A(7), (float *)A(8), (float *)A(9), A(10), n - 256, 1, 256, 256, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_WORKSPACE, "bwd short workspace", rc);
        rc = nsa_sel_bwd(in[0], in[1], in[2], (const int32_t *)in[3], in[4], (const float *)in[5], in[6],
                         (float *)A(7), (float *)A(8), (float *)A(9), A(0), n, 1, 256, 256, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_ALIAS, "bwd workspace alias", rc);
        rc = nsa_sel_bwd_noalloc(in[0], in[1], in[2], (const int32_t *)in[3], in[4], (const float *)in[5], in[6],
                                 (float *)A(7), (float *)A(8), (float *)A(9), 1, 65536, 65536, 64, 8, 128, 64, 16, 0);
        expect(rc == NSA_SEL_ERR_SCRATCH, "bwd noalloc scratch", rc);
        rc = nsa_sel_bwd_noalloc(nullptr, in[1], in[2], (const int32_t *)in[3], in[4], (const float *)in[5], in[6],
                                 (float *)A(7), (float *)A(8), (float *)A(9), 1, 64, 64, 8, 2, 64, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_NULL, "bwd noalloc null", rc);
    }
    // top-k
    {
        int rc = nsa_topk_blocks((const float *)A(0), nullptr, 1, 64, 2, 2, 32, 4, 0);
        expect(rc == NSA_SEL_ERR_NULL, "topk null", rc);
        rc = nsa_topk_blocks((const float *)A(0), (int32_t *)A(1), 1, 64, 2, 0, 32, 4, 0);
        expect(rc != NSA_SEL_OK, "topk shape", rc);
    }
    for (int s = -1; s < 12; ++s) expect(strlen(nsa_sel_status_string(s)) > 0, "status string", s);
    if (failures) return 1;
    printf("host checks: ok\n");
    return 0;
}
