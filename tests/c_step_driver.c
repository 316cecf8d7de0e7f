/*
 * One rank's step driven from plain C through the library's C ABI: reduce the
 * rank's slice from nd contributions, take the global norm and clip
 * multiplier, run AdamW on the fp32 state and write the 16-bit parameters.
 * Device memory comes from hipMalloc; nothing but this program and the
 * library touches the GPU.
 *
 * Usage: c_step_driver DIR N ND DTYPE
 *   reads  DIR/contribs.bin (ND x N 16-bit values, rank-major), DIR/master.bin,
 *          DIR/m.bin, DIR/v.bin (N fp32 each)
 *   writes DIR/out_reduced.bin, DIR/out_master.bin, DIR/out_m.bin,
 *          DIR/out_v.bin, DIR/out_param.bin, DIR/out_scalars.bin
 *          (norm as fp64, then clip multiplier as fp32, then flag as int32)
 * Test fixture: compiled and run by tests/test_gpu_c_driver.py.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_flat.h"

static void die(const char* what) {
    fprintf(stderr, "c_step_driver: %s\n", what);
    exit(1);
}

static void check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "c_step_driver: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void check_zero(int rc, const char* what) {
    if (rc != ZERO_OK) {
        fprintf(stderr, "c_step_driver: %s returned %d: %s\n", what, rc, zero_last_error());
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

static void* device_copy(const void* host, size_t bytes) {
    void* d = NULL;
    check_hip(hipMalloc(&d, bytes), "hipMalloc");
    if (host) check_hip(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
    return d;
}

static void host_copy(const char* dir, const char* name, const void* dev, size_t bytes) {
    void* h = malloc(bytes);
    if (!h) die("malloc");
    check_hip(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
    write_file(dir, name, h, bytes);
    free(h);
}

int main(int argc, char** argv) {
    if (argc != 5) die("usage: c_step_driver DIR N ND DTYPE");
    const char* dir = argv[1];
    const int64_t n = atoll(argv[2]);
    const int nd = atoi(argv[3]);
    const int dtype = atoi(argv[4]);
    if (n <= 0 || nd < 1 || nd > ZERO_MAX_RANKS) die("bad N or ND");

    const size_t b16 = (size_t)n * 2, b32 = (size_t)n * 4;
    uint16_t* contribs = read_file(dir, "contribs.bin", b16 * (size_t)nd);
    float* master = read_file(dir, "master.bin", b32);
    float* m = read_file(dir, "m.bin", b32);
    float* v = read_file(dir, "v.bin", b32);

    const void** d_contribs = malloc(sizeof(void*) * (size_t)nd);
    if (!d_contribs) die("malloc");
    for (int r = 0; r < nd; ++r) d_contribs[r] = device_copy(contribs + (size_t)r * (size_t)n, b16);
    void* d_reduced = device_copy(NULL, b16);
    const int64_t ws_bytes = zero_workspace_bytes(n, 1);
    if (ws_bytes < 0) die("zero_workspace_bytes");
    void* d_ws = device_copy(NULL, (size_t)ws_bytes);
    const int32_t zero = 0;
    int32_t* d_flag = device_copy(&zero, 4);
    double* d_norm = device_copy(NULL, 8);
    float* d_coef = device_copy(NULL, 4);
    float* d_master = device_copy(master, b32);
    float* d_m = device_copy(m, b32);
    float* d_v = device_copy(v, b32);
    void* d_param = device_copy(NULL, b16);

    const zero_adam_hparams hp = {3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, 1};
    check_zero(zero_reduce_shard(d_contribs, nd, n, dtype, 1.0f, d_reduced, d_ws, ws_bytes, 0, d_flag, NULL),
               "zero_reduce_shard");
    check_zero(zero_grad_norm(NULL, n, dtype, 1.0f, d_ws, ws_bytes, 1, NULL, 0, 1.0f, d_flag, d_norm, d_coef, NULL),
               "zero_grad_norm");
    check_zero(zero_adam_step(d_master, d_m, d_v, d_reduced, dtype, n, &hp, d_coef, d_flag, d_param, dtype, NULL),
               "zero_adam_step");
    check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");

    host_copy(dir, "out_reduced.bin", d_reduced, b16);
    host_copy(dir, "out_master.bin", d_master, b32);
    host_copy(dir, "out_m.bin", d_m, b32);
    host_copy(dir, "out_v.bin", d_v, b32);
    host_copy(dir, "out_param.bin", d_param, b16);
    unsigned char scalars[16];
    check_hip(hipMemcpy(scalars, d_norm, 8, hipMemcpyDeviceToHost), "norm");
    check_hip(hipMemcpy(scalars + 8, d_coef, 4, hipMemcpyDeviceToHost), "coef");
    check_hip(hipMemcpy(scalars + 12, d_flag, 4, hipMemcpyDeviceToHost), "flag");
    write_file(dir, "out_scalars.bin", scalars, sizeof scalars);

    for (int r = 0; r < nd; ++r) check_hip(hipFree((void*)d_contribs[r]), "hipFree");
    void* bufs[] = {d_reduced, d_ws, d_flag, d_norm, d_coef, d_master, d_m, d_v, d_param};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) check_hip(hipFree(bufs[i]), "hipFree");
    free(d_contribs);
    free(contribs);
    free(master);
    free(m);
    free(v);
    printf("ok\n");
    return 0;
}
