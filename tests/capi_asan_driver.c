/* Host-side argument checks of every libmoonep entry point, run under AddressSanitizer.
 * Every call here is rejected (or answered) on the host before anything touches a GPU: bad or
 * NULL dims, NULL and misaligned pointers, unsupported flags, workspace sizes at the extremes of
 * the accepted dims.  Exits 0 when every code is the one the header documents. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moonep.h"

static int fails = 0;
#define EXPECT(call, code)                                                              \
    do {                                                                                \
        int rc_ = (call);                                                               \
        if (rc_ != (code)) {                                                            \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, \
                    (int)(code));                                                       \
            ++fails;                                                                    \
        }                                                                               \
    } while (0)

static moonep_dims_t dims(int R, int E, int B, int S, int K, int H, int I, unsigned flags) {
    moonep_dims_t d;
    memset(&d, 0, sizeof d);
    d.R = R; d.E = E; d.B = B; d.S = S; d.K = K; d.H = H; d.I = I; d.flags = flags;
    return d;
}

int main(void) {
    void* g = (void*)(uintptr_t)0x10000;        /* aligned, never dereferenced on the host */
    void* mis = (void*)(uintptr_t)0x10004;
    const int32_t* gi = (const int32_t*)g;
    int32_t* go = (int32_t*)g;
    float* gf = (float*)g;
    moonep_dims_t d = dims(8, 256, 4, 4096, 8, 7168, 2048, 0);

    /* workspace sizes over the whole accepted range, and 0 for invalid dims */
    static const int Rs[] = {1, 2, 8, 64}, Es[] = {64, 256, 1024}, Ss[] = {1, 63, 64, 4096, 65536};
    for (unsigned i = 0; i < sizeof Rs / sizeof *Rs; ++i)
        for (unsigned j = 0; j < sizeof Es / sizeof *Es; ++j)
            for (unsigned k = 0; k < sizeof Ss / sizeof *Ss; ++k) {
                moonep_dims_t x = dims(Rs[i], Es[j], 64, Ss[k], 16, 8, 0, 0);
                size_t n = moonep_plan_workspace_bytes(&x);
                int valid = Es[j] % Rs[i] == 0 && Es[j] / Rs[i] <= 64;
                if ((n != 0) != valid) {
                    fprintf(stderr, "workspace bytes %zu for R%d E%d S%d\n", n, Rs[i], Es[j], Ss[k]);
                    ++fails;
                }
            }
    if (moonep_plan_workspace_bytes(NULL) != 0) ++fails;

    /* planning */
    EXPECT(moonep_plan(NULL, gi, g, go, go, go, NULL), MOONEP_EINVAL);
    EXPECT(moonep_plan(&d, NULL, g, go, go, go, NULL), MOONEP_EINVAL);
    EXPECT(moonep_plan(&d, gi, NULL, go, go, go, NULL), MOONEP_EINVAL);
    EXPECT(moonep_plan(&d, (const int32_t*)mis, g, go, go, go, NULL), MOONEP_EALIGN);
    moonep_dims_t bad = dims(8, 255, 4, 4096, 8, 7168, 0, 0);
    EXPECT(moonep_plan(&bad, gi, g, go, go, go, NULL), MOONEP_EINVAL);
    bad = dims(8, 256, 4, 4096, 17, 7168, 0, 0);
    EXPECT(moonep_plan(&bad, gi, g, go, go, go, NULL), MOONEP_EINVAL);
    bad = dims(8, 256, 4, 4096, 8, 7168, 0, 1u << 20);
    EXPECT(moonep_plan(&bad, gi, g, go, go, go, NULL), MOONEP_EINVAL);

    /* allocation-free planning: checks first, and dims beyond its static workspace */
    EXPECT(moonep_plan_noalloc(NULL, gi, go, go, go, NULL), MOONEP_EINVAL);
    EXPECT(moonep_plan_noalloc(&d, gi, go, (int32_t*)mis, go, NULL), MOONEP_EALIGN);
    moonep_dims_t huge = dims(16, 1024, 4, 65536, 8, 128, 0, 0);
    EXPECT(moonep_plan_noalloc(&huge, gi, go, go, go, NULL), MOONEP_ETOOBIG);

    /* permute / unpermute, staged forms */
    EXPECT(moonep_dispatch(&d, NULL, g, NULL, g, NULL), MOONEP_EINVAL);
    EXPECT(moonep_dispatch(&d, gi, mis, NULL, g, NULL), MOONEP_EALIGN);
    EXPECT(moonep_dispatch(&d, gi, g, (const float*)mis, g, NULL), MOONEP_EALIGN);
    EXPECT(moonep_combine(&d, gi, g, NULL, NULL, NULL), MOONEP_EINVAL);
    bad = dims(8, 256, 4, 4096, 8, 12, 0, 0);
    EXPECT(moonep_combine(&bad, gi, g, NULL, g, NULL), MOONEP_EINVAL);
    EXPECT(moonep_dispatch_staged(&d, gi, g, NULL, NULL, g, NULL), MOONEP_EINVAL);
    EXPECT(moonep_combine_staged(&d, gi, g, NULL, g, mis, NULL), MOONEP_EALIGN);

    /* expert FFN */
    moonep_dims_t f32 = dims(8, 256, 4, 4096, 8, 7168, 2048, MOONEP_F32_ROWS);
    EXPECT(moonep_grouped_ffn(&f32, g, gi, g, g, g, g, g, g, g, g, NULL), MOONEP_ENOTSUP);
    moonep_dims_t odd = dims(8, 256, 4, 4096, 8, 7176, 2048, 0);
    EXPECT(moonep_grouped_ffn(&odd, g, gi, g, g, g, g, g, g, g, g, NULL), MOONEP_ENOTSUP);
    moonep_dims_t noi = dims(8, 256, 4, 4096, 8, 7168, 0, 0);
    EXPECT(moonep_grouped_ffn(&noi, g, gi, g, g, g, g, g, g, g, g, NULL), MOONEP_EINVAL);
    EXPECT(moonep_grouped_ffn(&d, g, gi, g, g, g, g, g, mis, g, g, NULL), MOONEP_EALIGN);
    EXPECT(moonep_grouped_ffn_backward(&d, g, gi, g, NULL, g, g, g, g, g, g, g, gf, gf, gf, gf, NULL),
           MOONEP_EINVAL);
    EXPECT(moonep_grouped_ffn_backward(&d, g, gi, g, g, g, g, g, g, g, g, g, gf, gf, gf, (float*)mis, NULL),
           MOONEP_EALIGN);

    /* weights */
    EXPECT(moonep_prefetch(&d, NULL, g, g, g, g, NULL), MOONEP_EINVAL);
    EXPECT(moonep_prefetch(&d, g, g, g, NULL, g, NULL), MOONEP_EINVAL);
    EXPECT(moonep_reduce_grad(&d, g, gf, gf, gf, (float*)mis, NULL), MOONEP_EALIGN);
    EXPECT(moonep_reduce_grad(&noi, g, gf, gf, gf, gf, NULL), MOONEP_EINVAL);

    /* strings */
    for (int c = -6; c <= 1; ++c)
        if (!moonep_strerror(c) || !moonep_strerror(c)[0]) ++fails;
    if (!strstr(moonep_version(), "gfx950")) ++fails;

    if (fails) {
        fprintf(stderr, "%d host checks failed\n", fails);
        return 1;
    }
    printf("host checks passed\n");
    return 0;
}
