/*
 * abi_consumer.c -- a plain C11 caller of the fused MoE layer's C ABI
 * (include/moe.h), with no Python and no torch: device memory from the HIP
 * runtime, one moe_fused_forward call on the null stream, y copied back.
 *
 * usage: abi_consumer DIR T H I E K
 *   reads  DIR/x.bin (bf16 [T][H]), DIR/topk_idx.bin (int64 [T][K]),
 *          DIR/topk_w.bin (fp32 [T][K]), DIR/W1q.bin, DIR/S1.bin, DIR/W2q.bin,
 *          DIR/S2.bin (the layouts include/moe.h documents)
 *   writes DIR/y.bin (bf16 [T][H])
 * Exit status 0 on success; otherwise the failing step and status are printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "abi_consumer: cannot open %s\n", path);
        return NULL;
    }
    void* p = malloc(bytes ? bytes : 1);
    const size_t got = p ? fread(p, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        fprintf(stderr, "abi_consumer: %s holds %zu bytes, expected %zu\n", path, got, bytes);
        free(p);
        return NULL;
    }
    return p;
}

/* host buffer -> new device buffer */
static void* upload(const void* host, size_t bytes) {
    void* d = NULL;
    if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess) return NULL;
    if (bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(d);
        return NULL;
    }
    return d;
}

int main(int argc, char** argv) {
    if (argc != 7) {
        fprintf(stderr, "usage: %s DIR T H I E K\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    moe_shape_t s;
    s.T = atoi(argv[2]);
    s.H = atoi(argv[3]);
    s.I = atoi(argv[4]);
    s.E = atoi(argv[5]);
    s.K = atoi(argv[6]);
    const size_t T = (size_t)s.T, H = (size_t)s.H, I = (size_t)s.I, E = (size_t)s.E, K = (size_t)s.K;
    const size_t bytes[7] = {T * H * 2,          T * K * 8,          T * K * 4,
                             E * 2 * I * H / 2,  E * 2 * I * H / 32, E * H * I / 2,
                             E * H * I / 32};
    const char* names[7] = {"x.bin", "topk_idx.bin", "topk_w.bin", "W1q.bin",
                            "S1.bin", "W2q.bin", "S2.bin"};
    void* host[7];
    void* dev[7];
    for (int i = 0; i < 7; ++i) {
        host[i] = read_file(dir, names[i], bytes[i]);
        if (!host[i]) return 1;
        dev[i] = upload(host[i], bytes[i]);
        if (!dev[i]) {
            fprintf(stderr, "abi_consumer: device copy of %s failed\n", names[i]);
            return 1;
        }
    }
    const size_t ws_bytes = moe_workspace_bytes(&s);
    void *ws = NULL, *y = NULL;
    if (hipMalloc(&ws, ws_bytes) != hipSuccess || hipMalloc(&y, T * H * 2) != hipSuccess) {
        fprintf(stderr, "abi_consumer: hipMalloc of the workspace (%zu bytes) or y failed\n", ws_bytes);
        return 1;
    }
    const int rc = moe_fused_forward(&s, NULL, dev[0], (const int64_t*)dev[1], (const float*)dev[2],
                                     (const uint8_t*)dev[3], (const uint8_t*)dev[4],
                                     (const uint8_t*)dev[5], (const uint8_t*)dev[6], y, ws,
                                     ws_bytes, NULL);
    if (rc != MOE_OK) {
        fprintf(stderr, "abi_consumer: moe_fused_forward: %s (%d)\n", moe_status_string(rc), rc);
        return 1;
    }
    void* y_host = malloc(T * H * 2 + 1);
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(y_host, y, T * H * 2, hipMemcpyDeviceToHost) != hipSuccess) {
        fprintf(stderr, "abi_consumer: the forward call or the copy back failed\n");
        return 1;
    }
    char path[4096];
    snprintf(path, sizeof path, "%s/y.bin", dir);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(y_host, 1, T * H * 2, f) != T * H * 2) {
        fprintf(stderr, "abi_consumer: cannot write %s\n", path);
        return 1;
    }
    fclose(f);
    for (int i = 0; i < 7; ++i) {
        (void)hipFree(dev[i]);
        free(host[i]);
    }
    (void)hipFree(ws);
    (void)hipFree(y);
    free(y_host);
    printf("abi_consumer: T=%d H=%d I=%d E=%d K=%d ok (workspace %zu bytes)\n", s.T, s.H, s.I, s.E,
           s.K, ws_bytes);
    return 0;
}
