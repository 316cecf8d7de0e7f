/*
 * Every rank of a data-parallel group on one GPU, stepped from plain C through
 * the library's C ABI, the step captured once in a HIP graph and replayed.
 *
 * The flat vector of PSI parameters is partitioned over ND ranks (ZeRO-2, one
 * unit) with zero_plan_create.  Each step: zero_reduce_owners (every owner's
 * slice in one launch), zero_grad_norm (finalize over every owner's partial
 * sums), zero_adam_step_owners (every owner's AdamW in one launch, its scalars
 * from a device table indexed by the device step count) and zero_step_end.
 * Step 1 runs eagerly; the same four calls are then captured once on a
 * stream and the graph is launched for steps 2 and 3, each after the host has
 * copied that step's gradients into the (fixed) local gradient buffers.
 *
 * Usage: c_graph_driver DIR PSI ND DTYPE
 *   reads  DIR/grads.bin (3 steps x ND ranks x PSI 16-bit values, step-major,
 *          then rank-major), DIR/master.bin, DIR/m.bin, DIR/v.bin (ND x n fp32,
 *          owner-major, n the padded slice length of the plan)
 *   writes DIR/out_master.bin, DIR/out_m.bin, DIR/out_v.bin (ND x n fp32),
 *          DIR/out_param.bin (the padded full 16-bit parameter vector) and
 *          DIR/out_state.bin (the zero_step_state)
 * Test fixture: compiled and run by tests/test_gpu_c_driver.py.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_flat.h"

#define STEPS 3
#define TABLE_LEN 8

static void die(const char* what) {
    fprintf(stderr, "c_graph_driver: %s\n", what);
    exit(1);
}

static void check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "c_graph_driver: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void check_zero(int rc, const char* what) {
    if (rc != ZERO_OK) {
        fprintf(stderr, "c_graph_driver: %s returned %d: %s\n", what, rc, zero_last_error());
        exit(1);
    }
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) die(path);
    void* buf = malloc(bytes);
    if (!buf || fread(buf, 1, bytes, f) != bytes) die(path);
    fclose(f);
    return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes) die(path);
    fclose(f);
}

static void* device_alloc(size_t bytes) {
    void* d = NULL;
    check_hip(hipMalloc(&d, bytes), "hipMalloc");
    check_hip(hipMemset(d, 0, bytes), "hipMemset");
    return d;
}

static void host_copy(const char* dir, const char* name, const void* dev, size_t bytes) {
    void* h = malloc(bytes);
    if (!h) die("malloc");
    check_hip(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
    write_file(dir, name, h, bytes);
    free(h);
}

/* Step k's local gradients into rank r's buffer: PSI values, the padding stays zero. */
static void load_gradients(const uint16_t* grads, int k, int nd, int64_t psi, uint16_t* const* d_local) {
    for (int r = 0; r < nd; ++r)
        check_hip(hipMemcpy(d_local[r], grads + ((size_t)k * (size_t)nd + (size_t)r) * (size_t)psi,
                            (size_t)psi * 2, hipMemcpyHostToDevice),
                  "gradients to the device");
}

int main(int argc, char** argv) {
    if (argc != 5) die("usage: c_graph_driver DIR PSI ND DTYPE");
    const char* dir = argv[1];
    const int64_t psi = atoll(argv[2]);
    const int nd = atoi(argv[3]);
    const int dtype = atoi(argv[4]);
    if (psi <= 0 || nd < 2 || nd > 64) die("bad PSI or ND (2..64 ranks)");

    zero_plan* plan = NULL;
    check_zero(zero_plan_create(&psi, 1, nd, 2, 8, &plan), "zero_plan_create");
    int64_t n = 0, real = 0, full = 0;
    check_zero(zero_plan_rank(plan, 0, &n, &real), "zero_plan_rank");
    check_zero(zero_plan_full_numel(plan, &full), "zero_plan_full_numel");

    const size_t state_bytes = (size_t)nd * (size_t)n * 4;
    uint16_t* grads = read_file(dir, "grads.bin", (size_t)STEPS * (size_t)nd * (size_t)psi * 2);
    float* master = read_file(dir, "master.bin", state_bytes);
    float* m = read_file(dir, "m.bin", state_bytes);
    float* v = read_file(dir, "v.bin", state_bytes);

    /* Rank r's full local gradient: one row of an [nd, full] block; owner o's
     * contribution from rank r starts at o * n in that row. */
    uint16_t* d_block = device_alloc((size_t)nd * (size_t)full * 2);
    uint16_t** d_local = malloc(sizeof(uint16_t*) * (size_t)nd);
    const void** contribs = malloc(sizeof(void*) * (size_t)nd);
    if (!d_local || !contribs) die("malloc");
    for (int r = 0; r < nd; ++r) {
        d_local[r] = d_block + (size_t)r * (size_t)full;
        contribs[r] = d_local[r];
    }
    uint16_t* d_reduced = device_alloc((size_t)nd * (size_t)n * 2);
    const int64_t ws_bytes = zero_workspace_bytes(n, nd);
    if (ws_bytes < 0) die("zero_workspace_bytes");
    void* d_ws = device_alloc((size_t)ws_bytes);
    int32_t* d_flag = device_alloc(4);
    double* d_norm = device_alloc(8);
    float* d_coef = device_alloc(4);
    float* d_master = device_alloc(state_bytes);
    float* d_m = device_alloc(state_bytes);
    float* d_v = device_alloc(state_bytes);
    uint16_t* d_param = device_alloc((size_t)full * 2);
    check_hip(hipMemcpy(d_master, master, state_bytes, hipMemcpyHostToDevice), "master");
    check_hip(hipMemcpy(d_m, m, state_bytes, hipMemcpyHostToDevice), "m");
    check_hip(hipMemcpy(d_v, v, state_bytes, hipMemcpyHostToDevice), "v");

    /* AdamW's scalars for steps 1..TABLE_LEN, and the step state at t = 1. */
    zero_adam_consts table[TABLE_LEN];
    for (int t = 1; t <= TABLE_LEN; ++t) {
        const zero_adam_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1.0f, t};
        check_zero(zero_adam_consts_fill(&hp, &table[t - 1]), "zero_adam_consts_fill");
    }
    zero_adam_consts* d_table = device_alloc(sizeof table);
    check_hip(hipMemcpy(d_table, table, sizeof table, hipMemcpyHostToDevice), "table");
    const zero_step_state st0 = {1, 0, 0, 1, 0, 0};
    zero_step_state* d_state = device_alloc(sizeof st0);
    check_hip(hipMemcpy(d_state, &st0, sizeof st0, hipMemcpyHostToDevice), "state");

    hipStream_t s;
    check_hip(hipStreamCreate(&s), "hipStreamCreate");
#define ENQUEUE_STEP()                                                                                          \
    do {                                                                                                        \
        check_zero(zero_reduce_owners(contribs, nd, n, nd, n, dtype, 1.0f, d_reduced, n, d_ws, ws_bytes, d_flag, \
                                      s),                                                                       \
                   "zero_reduce_owners");                                                                       \
        check_zero(zero_grad_norm(NULL, n, dtype, 1.0f, d_ws, ws_bytes, nd, NULL, 0, 1.0f, d_flag, d_norm,     \
                                  d_coef, s),                                                                   \
                   "zero_grad_norm");                                                                           \
        check_zero(zero_adam_step_owners(d_master, d_m, d_v, n, d_reduced, dtype, n, n, nd, d_table, TABLE_LEN, \
                                         d_state, d_coef, d_flag, d_param, n, dtype, s),                        \
                   "zero_adam_step_owners");                                                                    \
        check_zero(zero_step_end(d_flag, d_state, s), "zero_step_end");                                        \
    } while (0)

    /* step 1, eagerly */
    load_gradients(grads, 0, nd, psi, d_local);
    ENQUEUE_STEP();
    check_hip(hipStreamSynchronize(s), "step 1");

    /* the same step, captured once */
    hipGraph_t graph;
    hipGraphExec_t exec;
    check_hip(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal), "hipStreamBeginCapture");
    ENQUEUE_STEP();
    check_hip(hipStreamEndCapture(s, &graph), "hipStreamEndCapture");
    check_hip(hipGraphInstantiate(&exec, graph, NULL, NULL, 0), "hipGraphInstantiate");

    /* steps 2 and 3: new gradients, then a replay */
    for (int k = 1; k < STEPS; ++k) {
        load_gradients(grads, k, nd, psi, d_local);
        check_hip(hipGraphLaunch(exec, s), "hipGraphLaunch");
        check_hip(hipStreamSynchronize(s), "replay");
    }

    host_copy(dir, "out_master.bin", d_master, state_bytes);
    host_copy(dir, "out_m.bin", d_m, state_bytes);
    host_copy(dir, "out_v.bin", d_v, state_bytes);
    host_copy(dir, "out_param.bin", d_param, (size_t)full * 2);
    host_copy(dir, "out_state.bin", d_state, sizeof st0);

    check_hip(hipGraphExecDestroy(exec), "hipGraphExecDestroy");
    check_hip(hipGraphDestroy(graph), "hipGraphDestroy");
    check_hip(hipStreamDestroy(s), "hipStreamDestroy");
    void* bufs[] = {d_block, d_reduced, d_ws, d_flag, d_norm, d_coef, d_master, d_m, d_v, d_param, d_table, d_state};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) check_hip(hipFree(bufs[i]), "hipFree");
    zero_plan_destroy(plan);
    free(d_local);
    free(contribs);
    free(grads);
    free(master);
    free(m);
    free(v);
    printf("ok\n");
    return 0;
}
