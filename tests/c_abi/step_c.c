/*
 * A plain C consumer of libzero_shard.so: no Python, no torch.  Reads a
 * problem from a binary file, runs zero_build_chunks + zero_shard_step (and
 * zero_shard_step_bf16_moments when asked) with hipMalloc'd buffers, and
 * writes the results to another binary file for comparison.
 *
 * State 2 runs the fp32-moment step from a HIP graph instead: the step with
 * its constants in a device table (zero_shard_step_scheduled) and the index
 * advance are captured once on a stream, and the graph is launched
 * GRAPH_STEPS + 1 times.  The table holds steps step .. step+GRAPH_STEPS-1,
 * so the launches apply those steps in turn and the last one, past the end
 * of the table, changes nothing; the final index is checked.
 *
 * Input file (little endian):  int32 n_ranks, int32 n_tensors, int32 rank,
 *   int32 state (0 = fp32 moments, 1 = bf16 moments, 2 = fp32 moments from a
 *   graph), int64 step,
 *   double lr, beta1, beta2, eps, weight_decay, int64 numels[n_tensors],
 *   then for shard length S: uint16 partials[n_ranks][S], float master[S],
 *   then m[S], v[S] as float (state 0) or uint16 (state 1).
 * Output file: float master[S], m[S], v[S] (float or uint16), uint16 params[S].
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_shard.h"

#define GRAPH_STEPS 4

#define CHECK_HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); exit(2); } } while (0)
#define CHECK_ZS(x) do { int r_ = (x); if (r_ != ZERO_OK) { \
    fprintf(stderr, "%s failed: %s\n", #x, zero_strerror(r_)); exit(3); } } while (0)

static void read_exact(FILE *f, void *p, size_t n)
{
    if (fread(p, 1, n, f) != n) { fprintf(stderr, "short read\n"); exit(4); }
}

int main(int argc, char **argv)
{
    if (argc != 3) { fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]); return 1; }
    FILE *in = fopen(argv[1], "rb");
    if (!in) { perror(argv[1]); return 1; }
    int32_t n_ranks, n_tensors, rank, state;
    int64_t step;
    double hpd[5];
    read_exact(in, &n_ranks, 4); read_exact(in, &n_tensors, 4);
    read_exact(in, &rank, 4); read_exact(in, &state, 4);
    read_exact(in, &step, 8); read_exact(in, hpd, sizeof hpd);
    int64_t *numels = malloc(sizeof(int64_t) * n_tensors);
    read_exact(in, numels, sizeof(int64_t) * n_tensors);

    int64_t n_chunks = 0, S = 0, total = 0;
    for (int t = 0; t < n_tensors; ++t) total += numels[t];
    /* parameter slot: this rank's part of one flat buffer */
    uint16_t *d_params = NULL;
    CHECK_HIP(hipMalloc((void **)&d_params, (size_t)total * 2 + 16));
    CHECK_ZS(zero_build_chunks(numels, n_tensors, n_ranks, rank, NULL, d_params, 2048,
                               NULL, 0, &n_chunks, &S));
    int64_t lo = (int64_t)rank * S < total ? (int64_t)rank * S : total;
    int64_t hi = lo + S < total ? lo + S : total;
    int64_t n = hi - lo;
    /* the slot starts at element lo of the flat buffer */
    CHECK_ZS(zero_build_chunks(numels, n_tensors, n_ranks, rank, NULL, d_params + lo, 2048,
                               NULL, 0, &n_chunks, &S));
    zero_chunk *table = malloc(sizeof(zero_chunk) * (n_chunks ? n_chunks : 1));
    CHECK_ZS(zero_build_chunks(numels, n_tensors, n_ranks, rank, NULL, d_params + lo, 2048,
                               table, n_chunks, &n_chunks, &S));

    size_t mom = state == 1 ? 2 : 4;
    uint16_t *h_parts = malloc((size_t)n_ranks * n * 2);
    float *h_master = malloc((size_t)n * 4);
    void *h_m = malloc((size_t)n * mom), *h_v = malloc((size_t)n * mom);
    read_exact(in, h_parts, (size_t)n_ranks * n * 2);
    read_exact(in, h_master, (size_t)n * 4);
    read_exact(in, h_m, (size_t)n * mom);
    read_exact(in, h_v, (size_t)n * mom);
    fclose(in);

    const void **parts = malloc(sizeof(void *) * n_ranks);
    for (int k = 0; k < n_ranks; ++k) {
        void *d = NULL;
        CHECK_HIP(hipMalloc(&d, (size_t)n * 2 + 16));
        CHECK_HIP(hipMemcpy(d, h_parts + (size_t)k * n, (size_t)n * 2, hipMemcpyHostToDevice));
        parts[k] = d;
    }
    float *d_master = NULL;
    void *d_m = NULL, *d_v = NULL;
    zero_chunk *d_table = NULL;
    CHECK_HIP(hipMalloc((void **)&d_master, (size_t)n * 4 + 16));
    CHECK_HIP(hipMalloc(&d_m, (size_t)n * mom + 16));
    CHECK_HIP(hipMalloc(&d_v, (size_t)n * mom + 16));
    CHECK_HIP(hipMalloc((void **)&d_table, sizeof(zero_chunk) * (n_chunks ? n_chunks : 1)));
    CHECK_HIP(hipMemcpy(d_master, h_master, (size_t)n * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_m, h_m, (size_t)n * mom, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_v, h_v, (size_t)n * mom, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_table, table, sizeof(zero_chunk) * n_chunks, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_params, 0xFF, (size_t)total * 2));
    {   /* the table against every array the step reads or writes */
        const void **arr = malloc(sizeof(void *) * (n_ranks + 3));
        int64_t *bytes = malloc(sizeof(int64_t) * (n_ranks + 3));
        for (int k = 0; k < n_ranks; ++k) {
            arr[k] = parts[k];
            bytes[k] = n * 2;
        }
        arr[n_ranks] = d_master, bytes[n_ranks] = n * 4;
        arr[n_ranks + 1] = d_m, bytes[n_ranks + 1] = n * (int64_t)mom;
        arr[n_ranks + 2] = d_v, bytes[n_ranks + 2] = n * (int64_t)mom;
        CHECK_ZS(zero_check_chunks(table, n_chunks, n, (const void *const *)arr, bytes, n_ranks + 3));
        free(arr);
        free(bytes);
    }

    zero_adamw_hparams hp = {hpd[0], hpd[1], hpd[2], hpd[3], hpd[4], step};
    if (state == 0) {
        CHECK_ZS(zero_shard_step(parts, n_ranks, ZERO_BF16, d_master, (float *)d_m, (float *)d_v,
                                 n, d_table, n_chunks, &hp, 0));
    } else if (state == 1) {
        CHECK_ZS(zero_shard_step_bf16_moments(parts, n_ranks, ZERO_BF16, d_master, (uint16_t *)d_m,
                                              (uint16_t *)d_v, n, d_table, n_chunks, &hp, 0));
    } else {
        zero_adamw_hparams hps[GRAPH_STEPS];
        zero_step_consts consts[GRAPH_STEPS];
        for (int i = 0; i < GRAPH_STEPS; ++i) {
            hps[i] = hp;
            hps[i].step = step + i;
        }
        CHECK_ZS(zero_make_step_consts(hps, GRAPH_STEPS, consts));
        zero_step_consts *d_consts = NULL;
        int64_t *d_index = NULL, index = 0;
        CHECK_HIP(hipMalloc((void **)&d_consts, sizeof consts));
        CHECK_HIP(hipMalloc((void **)&d_index, sizeof index));
        CHECK_HIP(hipMemcpy(d_consts, consts, sizeof consts, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(d_index, &index, sizeof index, hipMemcpyHostToDevice));
        hipStream_t stream;
        hipGraph_t graph;
        hipGraphExec_t exec;
        CHECK_HIP(hipStreamCreate(&stream));
        CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
        CHECK_ZS(zero_shard_step_scheduled(parts, n_ranks, ZERO_BF16, d_master, (float *)d_m,
                                           (float *)d_v, n, d_table, n_chunks, d_consts,
                                           GRAPH_STEPS, d_index, stream));
        CHECK_ZS(zero_step_index_advance(d_index, GRAPH_STEPS, stream));
        CHECK_HIP(hipStreamEndCapture(stream, &graph));
        CHECK_HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
        for (int r = 0; r <= GRAPH_STEPS; ++r)
            CHECK_HIP(hipGraphLaunch(exec, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(&index, d_index, sizeof index, hipMemcpyDeviceToHost));
        if (index != GRAPH_STEPS) {
            fprintf(stderr, "index %lld after the launches, want %d\n", (long long)index, GRAPH_STEPS);
            return 5;
        }
        CHECK_HIP(hipGraphExecDestroy(exec));
        CHECK_HIP(hipGraphDestroy(graph));
        CHECK_HIP(hipStreamDestroy(stream));
        CHECK_HIP(hipFree(d_consts));
        CHECK_HIP(hipFree(d_index));
    }
    CHECK_HIP(hipDeviceSynchronize());

    uint16_t *h_params = malloc((size_t)total * 2);
    CHECK_HIP(hipMemcpy(h_master, d_master, (size_t)n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_m, d_m, (size_t)n * mom, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_v, d_v, (size_t)n * mom, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_params, d_params, (size_t)total * 2, hipMemcpyDeviceToHost));
    FILE *out = fopen(argv[2], "wb");
    if (!out) { perror(argv[2]); return 1; }
    fwrite(h_master, 4, (size_t)n, out);
    fwrite(h_m, mom, (size_t)n, out);
    fwrite(h_v, mom, (size_t)n, out);
    fwrite(h_params, 2, (size_t)total, out);
    fclose(out);
    printf("ok n=%lld chunks=%lld\n", (long long)n, (long long)n_chunks);
    return 0;
}
