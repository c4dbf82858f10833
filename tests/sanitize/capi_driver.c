/*
 * Exercises the host side of the C ABI in include/convfwd.h -- descriptor
 * validation, output extents, the tile-configuration selector, plan
 * creation and description for every compiled configuration, the fused
 * chain and backward plans, and the argument checks every run call makes
 * before it would launch -- in a build whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing here launches a
 * kernel: every run call below is refused by the library's own checks
 * (NULL or misaligned pointers), so the driver needs no GPU.  Prints
 * "capi sanitize ok" at the end.  Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "convfwd.h"

static int failures = 0;

#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, conv_fwd_last_error()); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static conv_fwd_desc_t desc(int ndim, int dt, int64_t N, int64_t G, int64_t C, int64_t K, int64_t D, int64_t H,
                            int64_t W, int64_t Z, int64_t Y, int64_t X, int64_t s, int64_t p, int64_t d, int bias,
                            int gelu)
{
    conv_fwd_desc_t r;
    memset(&r, 0, sizeof(r));
    r.ndim = ndim;
    r.dtype = dt;
    r.N = N; r.G = G; r.C = C; r.K = K;
    r.in[0] = D; r.in[1] = H; r.in[2] = W;
    r.filt[0] = Z; r.filt[1] = Y; r.filt[2] = X;
    for (int i = 0; i < 3; ++i) {
        const int used = i >= 3 - ndim;
        r.stride[i] = used ? s : 1;
        r.pad[i] = used ? p : 0;
        r.dilation[i] = used ? d : 1;
    }
    r.has_bias = bias;
    r.gelu = gelu;
    return r;
}

/* A plan's queries, then run calls that the host checks refuse. */
static void probe_plan(conv_fwd_plan_t *pl)
{
    int64_t o[3], flop = -1;
    EXPECT(conv_fwd_out_dims(pl, o) == CONV_OK);
    EXPECT(conv_fwd_useful_flop(pl, &flop) == CONV_OK && flop >= 0);
    EXPECT(strlen(conv_fwd_describe(pl)) > 0);
    char *odd = (char *)0x1008;   /* 8-byte aligned only: refused before any launch */
    EXPECT(conv_fwd_run(pl, NULL, odd, NULL, odd, NULL) != CONV_OK || flop == 0);   /* N = 0: a no-op */
    EXPECT(conv_fwd_run(pl, odd, odd, odd, odd, NULL) != CONV_OK);
    EXPECT(conv_fwd_run_events(pl, odd, NULL, NULL, odd, NULL, NULL, NULL) != CONV_OK);
}

int main(void)
{
    conv_fwd_desc_t probs[] = {
        desc(1, CONV_DT_F32, 1, 1, 80, 384, 1, 1, 3000, 1, 1, 3, 1, 1, 1, 1, 0),
        desc(1, CONV_DT_F32, 1, 1, 384, 384, 1, 1, 3000, 1, 1, 3, 2, 1, 1, 1, 1),
        desc(1, CONV_DT_BF16, 32, 1, 80, 384, 1, 1, 3000, 1, 1, 3, 1, 1, 1, 1, 1),
        desc(1, CONV_DT_BF16, 32, 1, 384, 384, 1, 1, 3000, 1, 1, 3, 2, 1, 1, 1, 1),
        desc(2, CONV_DT_BF16, 8, 4, 64, 64, 1, 56, 56, 1, 3, 3, 1, 1, 1, 0, 0),
        desc(3, CONV_DT_BF16, 2, 8, 32, 32, 16, 28, 28, 3, 3, 3, 1, 2, 2, 0, 0),
        desc(3, CONV_DT_F32, 2, 3, 5, 7, 5, 9, 8, 3, 2, 3, 2, 1, 2, 1, 1),
        desc(2, CONV_DT_BF16, 0, 2, 8, 8, 1, 10, 10, 1, 3, 3, 1, 1, 1, 0, 0),      /* empty batch */
        desc(1, CONV_DT_BF16, 3, 1, 3, 5, 1, 1, 77, 1, 1, 5, 2, 2, 1, 1, 0),       /* odd channels */
        desc(2, CONV_DT_F32, 5, 1, 32, 16, 1, 3, 3, 1, 3, 3, 1, 0, 1, 0, 0),       /* 1x1 output */
    };
    const int nprob = (int)(sizeof(probs) / sizeof(probs[0]));
    const int ncfg = conv_fwd_num_configs();
    EXPECT(ncfg > 0);
    for (int i = 0; i < nprob; ++i) {
        conv_fwd_plan_t *pl = NULL;
        EXPECT(conv_fwd_create(&probs[i], &pl) == CONV_OK);
        if (pl) probe_plan(pl);
        conv_fwd_destroy(pl);
        for (int c = 0; c < ncfg; ++c) {   /* every configuration: accepted, or refused with a status */
            conv_fwd_plan_t *q = NULL;
            conv_status_t st = conv_fwd_create_with_config(&probs[i], c, &q);
            EXPECT((st == CONV_OK) == (q != NULL));
            if (q) probe_plan(q);
            conv_fwd_destroy(q);
        }
        conv_bwd_data_plan_t *bd = NULL;
        conv_bwd_weight_plan_t *bw = NULL;
        conv_fwd_desc_t lin = probs[i];
        lin.has_bias = lin.gelu = 0;
        if (conv_bwd_data_create(&lin, &bd) == CONV_OK) {
            int64_t b = -1;
            EXPECT(conv_bwd_data_workspace_bytes(bd, &b) == CONV_OK && b >= 0);
            EXPECT(strlen(conv_bwd_data_describe(bd)) > 0);
            EXPECT(conv_bwd_data_run(bd, (void *)0x1008, (void *)0x1008, (void *)0x1008, (void *)0x1008, b, NULL) !=
                       CONV_OK || lin.N == 0);
        }
        conv_bwd_data_destroy(bd);
        if (conv_bwd_weight_create(&lin, &bw) == CONV_OK) {
            int64_t b = -1;
            EXPECT(conv_bwd_weight_workspace_bytes(bw, &b) == CONV_OK && b >= 0);
            EXPECT(strlen(conv_bwd_weight_describe(bw)) > 0);
            EXPECT(conv_bwd_weight_run(bw, NULL, NULL, (void *)0x1008, NULL, 0, NULL) != CONV_OK);
        }
        conv_bwd_weight_destroy(bw);
    }
    /* invalid descriptors: refused with a message, no plan */
    conv_fwd_desc_t bad[] = {
        desc(0, CONV_DT_F32, 1, 1, 1, 1, 1, 1, 8, 1, 1, 3, 1, 0, 1, 0, 0),
        desc(1, 7, 1, 1, 1, 1, 1, 1, 8, 1, 1, 3, 1, 0, 1, 0, 0),
        desc(1, CONV_DT_F32, -1, 1, 1, 1, 1, 1, 8, 1, 1, 3, 1, 0, 1, 0, 0),
        desc(1, CONV_DT_F32, 1, 0, 1, 1, 1, 1, 8, 1, 1, 3, 1, 0, 1, 0, 0),
        desc(1, CONV_DT_F32, 1, 1, 1, 1, 1, 1, 2, 1, 1, 5, 1, 0, 1, 0, 0),      /* empty output */
        desc(1, CONV_DT_F32, 1, 1, 1, 1, 1, 1, 8, 1, 1, 3, 0, 0, 1, 0, 0),      /* stride 0 */
        desc(1, CONV_DT_F32, 1, 1, 1, 1, 1, 1, 8, 1, 1, 3, 1, -1, 1, 0, 0),     /* negative pad */
        desc(1, CONV_DT_F32, 1, 1, 1, 1, 1, 1, 8, 1, 1, 3, 1, 0, 1, 2, 0),      /* has_bias not 0/1 */
        desc(1, CONV_DT_BF16, 1 << 20, 1, 4096, 1, 1, 1, 4096, 1, 1, 1, 1, 0, 1, 0, 0),   /* beyond 2^31 */
    };
    for (int i = 0; i < (int)(sizeof(bad) / sizeof(bad[0])); ++i) {
        conv_fwd_plan_t *pl = (conv_fwd_plan_t *)0x1;
        EXPECT(conv_fwd_create(&bad[i], &pl) != CONV_OK && pl == NULL);
        EXPECT(strlen(conv_fwd_last_error()) > 0);
    }
    conv_fwd_desc_t unused = probs[0];
    unused.in[1] = 2;   /* a 1-D problem with a non-trivial unused dim */
    conv_fwd_plan_t *pl = NULL;
    EXPECT(conv_fwd_create(&unused, &pl) == CONV_ERR_INVALID_ARG);
    EXPECT(conv_fwd_create(NULL, &pl) == CONV_ERR_INVALID_ARG);
    EXPECT(conv_fwd_create(&probs[0], NULL) == CONV_ERR_INVALID_ARG);
    EXPECT(conv_fwd_create_with_config(&probs[0], ncfg, &pl) != CONV_OK);
    EXPECT(conv_fwd_create_with_config(&probs[0], -1, &pl) != CONV_OK);
    EXPECT(conv_fwd_config_name(-1) == NULL && conv_fwd_config_name(ncfg) == NULL);
    for (int c = 0; c < ncfg; ++c) EXPECT(conv_fwd_config_name(c) != NULL && conv_fwd_config_dtype(c) >= 0);
    EXPECT(strcmp(conv_fwd_describe(NULL), "") == 0);
    conv_fwd_destroy(NULL);

    /* fused chains: the frontend at several input widths and lengths */
    static const int64_t c1s[] = {16, 80, 224, 352, 72};
    static const int64_t ls[] = {3000, 301, 2, 1};
    for (int a = 0; a < 5; ++a)
        for (int b = 0; b < 4; ++b) {
            conv_fwd_desc_t f = desc(1, CONV_DT_BF16, 2, 1, c1s[a], 384, 1, 1, ls[b], 1, 1, 3, 1, 1, 1, 1, 1);
            conv_fwd_desc_t s = desc(1, CONV_DT_BF16, 2, 1, 384, 384, 1, 1, ls[b], 1, 1, 3, 2, 1, 1, 1, 1);
            conv_chain_plan_t *ch = NULL;
            conv_status_t st = conv_chain_create(&f, &s, &ch);
            EXPECT((st == CONV_OK) == (c1s[a] % 16 == 0 && c1s[a] <= 352));
            if (!ch) continue;
            int64_t o[3], flop = -1, pb = -1;
            EXPECT(conv_chain_out_dims(ch, o) == CONV_OK && o[2] == (ls[b] - 1) / 2 + 1);
            EXPECT(conv_chain_useful_flop(ch, &flop) == CONV_OK && flop > 0);
            st = conv_chain_packed_bytes(ch, &pb);
            EXPECT(st == CONV_OK ? pb > 0 : c1s[a] > 224);
            EXPECT(strlen(conv_chain_describe(ch)) > 0);
            EXPECT(conv_chain_run(ch, (void *)0x1008, (void *)0x1008, (void *)0x1008, (void *)0x1008,
                                  (void *)0x1008, (void *)0x1008, NULL) != CONV_OK);
            EXPECT(conv_chain_run_packed(ch, (void *)0x1008, NULL, NULL, NULL, (void *)0x1008, NULL) != CONV_OK);
            EXPECT(conv_chain_pack_weights(ch, NULL, NULL, NULL, NULL) != CONV_OK);
            conv_chain_destroy(ch);
        }
    conv_chain_destroy(NULL);
    printf("%d problems x %d configurations; capi sanitize %s\n", nprob, ncfg, failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
