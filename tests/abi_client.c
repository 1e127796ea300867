/* A plain C99 client of the library: the header must compile as C and the host
 * planner must be callable without any Python or torch in between.  Builds the
 * hand-worked 8-head plan and prints the exported tables, one per line, for
 * the test to compare with its golden fixture; then checks a few status codes. */
#include <stdio.h>
#include <stdlib.h>

#include "sketchssm.h"
#include "sketchssm_measure.h"

static void print_row(const char* name, const int32_t* x, int n) {
    int i;
    printf("%s", name);
    for (i = 0; i < n; ++i) printf(" %d", (int)x[i]);
    printf("\n");
}

int main(void) {
    const int32_t rank[8] = {0, 6, 6, 9, 1, 0, 17, 6};
    const int32_t group[8] = {0, 0, 0, 0, 1, 1, 1, 1};
    sketchssm_shape sh;
    sketchssm_plan* plan = NULL;
    sketchssm_status st;
    int32_t frame_index[8], frame_row_off[9], z_row_off[9], bucket[8], order[8];
    int32_t frame_group[8], frame_rank[8], n_frames = 0;

    sh.B = 4; sh.H = 8; sh.K = 128; sh.V = 80; sh.W = 16; sh.G = 2;
    sh.basis_rows = 79; sh.rank_cap = 49; sh.kind = SKSSM_MAMBA2; sh.qkv = SKSSM_BF16;
    sh.kq_heads = 0;

    st = sketchssm_plan_create(&sh, rank, group, &plan);
    if (st != SKSSM_OK || plan == NULL) {
        printf("plan_create failed: %s\n", sketchssm_status_string(st));
        return 1;
    }
    st = sketchssm_plan_export(plan, frame_index, frame_row_off, z_row_off, bucket, order,
                               frame_group, frame_rank, &n_frames);
    if (st != SKSSM_OK) return 2;
    print_row("frame_index", frame_index, 8);
    print_row("frame_row_off", frame_row_off, n_frames + 1);
    print_row("z_row_off", z_row_off, 9);
    print_row("bucket", bucket, 8);
    print_row("order", order, 8);
    print_row("frame_group", frame_group, n_frames);
    print_row("frame_rank", frame_rank, n_frames);
    printf("z_elems %lu\n", (unsigned long)sketchssm_z_elems(plan));
    printf("frame_elems %lu\n", (unsigned long)sketchssm_frame_elems(plan));
    sketchssm_plan_destroy(plan);

    /* status codes, checked on the host before anything could be launched */
    plan = NULL;
    printf("null_out %d\n", (int)sketchssm_plan_create(&sh, rank, group, NULL));
    sh.V = 72;
    printf("bad_V %d\n", (int)sketchssm_plan_create(&sh, rank, group, &plan));
    sh.V = 80;
    {
        /* an explicit launch order: the planner's own, reversed among the sketch
           heads, is accepted; a dense head placed after a sketch head is not */
        int32_t ord[8], i, nd = 0, ns = 0;
        int32_t dense_idx[8], sketch_idx[8];
        for (i = 0; i < 8; ++i) {
            if (rank[order[i]] == 0) dense_idx[nd++] = order[i];
            else sketch_idx[ns++] = order[i];
        }
        for (i = 0; i < nd; ++i) ord[i] = dense_idx[i];
        for (i = 0; i < ns; ++i) ord[nd + i] = sketch_idx[ns - 1 - i];
        st = sketchssm_plan_create_ordered(&sh, rank, group, ord, &plan);
        if (st == SKSSM_OK) {
            int32_t got[8];
            sketchssm_plan_export(plan, NULL, NULL, NULL, NULL, got, NULL, NULL, NULL);
            print_row("ordered", got, 8);
            sketchssm_plan_destroy(plan);
            plan = NULL;
        }
        printf("ordered_status %d\n", (int)st);
        if (nd > 0 && ns > 0) {
            int32_t t = ord[0];
            ord[0] = ord[7];
            ord[7] = t;
            printf("ordered_dense_late %d\n", (int)sketchssm_plan_create_ordered(&sh, rank, group, ord, &plan));
        }
    }
    printf("flush_null_plan %d\n", (int)sketchssm_flush(NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                                        NULL, 0, NULL));
    printf("probe_null %d\n", (int)sketchssm_stream_probe(NULL, 4096 * 8, NULL, 0, 8, 1, 0, NULL));
    printf("status_text %s\n", sketchssm_status_string(SKSSM_EALIGN));
    return 0;
}
