// Sanitizer driver for liblinattn's host-side validation (test
// infrastructure): linked with la_api.hip built with AddressSanitizer and
// UndefinedBehaviorSanitizer on its host code, it calls every entry point
// with argument sets that host validation must reject (so nothing reaches a
// device) and the host queries over a sweep of shapes, checking the status
// each returns.  Exit status 0: no sanitizer report and every status as
// expected.  It needs no GPU.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "liblinattn.h"

static int failures = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

static la_problem prob(int B, int H, int N, int dk, int dv, la_dtype dt, la_phi_kind phi) {
    la_problem p;
    p.B = B; p.H = H; p.N = N; p.d_k = dk; p.d_v = dv; p.dtype = dt; p.phi = phi;
    p.m = 0; p.W = nullptr; p.map_param = 0; p.pos0 = 0;
    return p;
}

int main() {
    void *fake = reinterpret_cast<void *>(uintptr_t(0x100000));    // aligned, never dereferenced
    void *mis = reinterpret_cast<void *>(uintptr_t(0x100004));
    float *ff = static_cast<float *>(fake);
    la_problem p = prob(2, 3, 100, 64, 64, LA_BF16, LA_PHI_ELU1);
    // host queries over a sweep of shapes, every map and chunk
    const int chunks[] = {16, 32, 64, 128};
    size_t total = 0;
    for (int dt = 0; dt < 2; ++dt)
        for (int phi = 0; phi <= 5; ++phi)
            for (int d : {1, 5, 64, 127, 128})
                for (int N : {1, 63, 64, 1000, 16384})
                    for (int BH : {1, 7, 32, 300}) {
                        la_problem q = prob(BH, 1, N, d, d, (la_dtype)dt, (la_phi_kind)phi);
                        if (phi == LA_PHI_FAVOR || phi == LA_PHI_TRIG) { q.m = 16; q.W = ff; }
                        if (phi == LA_PHI_DPFP || phi == LA_PHI_COSFORMER) q.map_param = 1;
                        for (int c : chunks) {
                            total += la_workspace_bytes(&q, c) + la_backward_workspace_bytes(&q, c) +
                                     la_gla_workspace_bytes(&q, c) + la_delta_workspace_bytes(&q, c);
                        }
                        total += (size_t)la_feature_dim(&q);
                    }
    expect(total > 0, 1, "workspace queries");
    expect(la_workspace_bytes(nullptr, 64) == 0, 1, "NULL problem");
    // rejections, one per rule
    expect(la_forward_causal_chunked(&p, 64, nullptr, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fake,
                                     1 << 30, nullptr), LA_ERR_NULL, "causal NULL Q");
    expect(la_forward_causal_chunked(&p, 48, fake, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fake,
                                     1 << 30, nullptr), LA_ERR_UNSUPPORTED, "causal chunk");
    expect(la_forward_causal_chunked(&p, 64, mis, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fake,
                                     1 << 30, nullptr), LA_ERR_ALIGN, "causal align");
    expect(la_forward_causal_chunked(&p, 64, fake, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fake, 0,
                                     nullptr), LA_ERR_WORKSPACE, "causal workspace");
    la_problem bad = prob(0, 3, 100, 64, 64, LA_BF16, LA_PHI_ELU1);
    expect(la_forward_causal_chunked(&bad, 64, fake, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fake,
                                     1 << 30, nullptr), LA_ERR_SHAPE, "causal shape");
    la_problem big = prob(255, 1, 256, 128, 128, LA_BF16, LA_PHI_ELU1);
    expect(la_forward_causal_chunked_noalloc(&big, 128, fake, fake, fake, fake, nullptr, nullptr, nullptr, nullptr,
                                             nullptr), LA_ERR_SCRATCH, "noalloc scratch");
    expect(la_forward_noncausal(&p, fake, fake, mis, fake, nullptr, nullptr, fake, 1 << 30, nullptr), LA_ERR_ALIGN,
           "noncausal align");
    la_problem p1 = prob(2, 3, 1, 64, 64, LA_F32, LA_PHI_ELU1);
    expect(la_decode_step(&p1, fake, fake, fake, fake, ff, static_cast<float *>(mis), nullptr), LA_ERR_ALIGN,
           "decode align");
    expect(la_decode_step(&p, fake, fake, fake, fake, ff, ff, nullptr), LA_ERR_SHAPE, "decode N");
    la_problem pid = prob(2, 3, 100, 64, 64, LA_BF16, LA_PHI_IDENTITY);
    expect(la_forward_retention_chunked(&pid, nullptr, 64, fake, fake, fake, fake, nullptr, nullptr, fake, 1 << 30,
                                        nullptr, nullptr), LA_ERR_NULL, "retention gamma");
    expect(la_retention_decode_step(&pid, ff, fake, fake, fake, fake, ff, nullptr), LA_ERR_SHAPE, "retention decode N");
    expect(la_backward_causal_chunked(&p, 64, fake, fake, fake, mis, nullptr, nullptr, nullptr, nullptr, fake, fake,
                                      fake, nullptr, nullptr, fake, 1 << 30, nullptr, nullptr), LA_ERR_ALIGN,
           "backward align");
    expect(la_forward_gla_recurrent(&p, fake, fake, fake, ff, nullptr, nullptr, fake, nullptr), LA_ERR_UNSUPPORTED,
           "gla map");
    expect(la_forward_delta_recurrent(&pid, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fake, nullptr),
           LA_ERR_NULL, "delta beta");
    expect(la_forward_gla_chunked(&pid, 64, fake, fake, fake, ff, nullptr, nullptr, fake, fake, 0, nullptr, nullptr),
           LA_ERR_WORKSPACE, "gla workspace");
    expect(la_forward_delta_chunked(&pid, 32, fake, fake, fake, nullptr, ff, nullptr, nullptr, fake, fake, 1 << 30,
                                    nullptr, nullptr), LA_ERR_UNSUPPORTED, "delta chunk");
    unsigned int *err = static_cast<unsigned int *>(fake);
    expect(la_workspace_error(fake, 255, err, 1, nullptr), LA_ERR_WORKSPACE, "error word size");
    for (int s = 0; s <= 9; ++s) expect(la_status_string((la_status)s) != nullptr, 1, "status string");
    expect(la_abi_version(), LA_ABI_VERSION, "abi version");
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("validation driver: all statuses as expected\n");
    return 0;
}
