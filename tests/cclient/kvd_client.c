/*
 * kvd_client.c -- a plain C caller of libkvd.so (tests only).
 *
 * Drives the C ABI of include/kvd.h with the HIP runtime and nothing else:
 * device and pinned host memory from hipMalloc / hipHostMalloc, one compute
 * stream, no Python.  Inputs come from files that the test writes with the
 * seeded input module; outputs go back to files for the test to check.
 *
 *   kvd_client DIR N_LAYERS N_ROWS N_HEAD_Q N_HEAD_KV HEAD_DIM
 *
 * DIR/k.bin, DIR/v.bin  uint8 [N_LAYERS][N_ROWS][row bytes]  q8_0 rows
 * DIR/q.bin             fp32  [N_LAYERS][N_HEAD_Q][HEAD_DIM]
 *
 * Writes
 * DIR/out_device.bin    layer 0 attended from device memory (kvd_attend_decode)
 * DIR/out_ring_d0.bin   every layer, host-resident K/V through a depth-0 ring
 * DIR/out_ring_d1.bin   the same through a depth-1 ring (prefetch one layer ahead)
 * and prints the depth-1 ring's counters.  Each ring arm runs two decode
 * steps over the stack (the second step's outputs are written); the stable
 * prefix is every row but the newest.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvd.h"

#define HIP_OK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                     \
        }                                                                                \
    } while (0)

#define KVD_OK_OR_DIE(call)                                                              \
    do {                                                                                 \
        int r_ = (call);                                                                 \
        if (r_ < 0) {                                                                    \
            fprintf(stderr, "%s:%d %s -> %d: %s\n", __FILE__, __LINE__, #call, r_, kvd_last_error()); \
            exit(3);                                                                     \
        }                                                                                \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(4);
    }
    void* p = malloc(bytes);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short read of %s (%zu bytes expected)\n", path, bytes);
        exit(4);
    }
    fclose(f);
    return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(4);
    }
    fclose(f);
}

/* One attention call over rows [0, n_rows) of one layer at (k, v). */
static void attend(const float* q, float* out, const void* k, const void* v, int64_t n_rows, int64_t stride,
                   int n_head_q, int n_head_kv, int head_dim, void** ws, size_t* ws_bytes, hipStream_t s) {
    kvd_kv_seg seg;
    memset(&seg, 0, sizeof seg);
    seg.k = k;
    seg.v = v;
    seg.n_rows = n_rows;
    seg.pos0 = 0;
    seg.row_stride = stride;
    kvd_attn_args a;
    memset(&a, 0, sizeof a);
    a.n_seq = 1;
    a.n_head_q = n_head_q;
    a.n_head_kv = n_head_kv;
    a.head_dim = head_dim;
    a.n_seg = 1;
    a.scale = 1.0f / sqrtf((float)head_dim);
    a.q = q;
    a.out = out;
    a.segs = &seg;
    a.v_type = KVD_TYPE_Q8_0;
    size_t need = 0;
    KVD_OK_OR_DIE(kvd_attend_workspace_bytes(&a, &need));
    if (need > *ws_bytes) {
        /* grow: nothing in flight may still use the old buffer */
        HIP_OK(hipStreamSynchronize(s));
        if (*ws) HIP_OK(hipFree(*ws));
        HIP_OK(hipMalloc(ws, need));
        *ws_bytes = need;
    }
    a.workspace = *ws;
    a.workspace_bytes = *ws_bytes;
    KVD_OK_OR_DIE(kvd_attend_decode(&a, s));
}

int main(int argc, char** argv) {
    if (argc != 7) {
        fprintf(stderr, "usage: %s DIR N_LAYERS N_ROWS N_HEAD_Q N_HEAD_KV HEAD_DIM\n", argv[0]);
        return 1;
    }
    const char* dir = argv[1];
    const int n_layers = atoi(argv[2]);
    const int64_t n_rows = atoll(argv[3]);
    const int n_head_q = atoi(argv[4]);
    const int n_head_kv = atoi(argv[5]);
    const int head_dim = atoi(argv[6]);
    if (n_layers < 1 || n_layers > 64 || n_rows < 2 || n_rows > (1 << 20) || head_dim % 32) {
        fprintf(stderr, "arguments out of range\n");
        return 1;
    }
    const int64_t row_bytes = (int64_t)n_head_kv * head_dim / 32 * 34;
    const size_t layer_bytes = (size_t)n_rows * (size_t)row_bytes;
    const size_t q_floats = (size_t)n_head_q * head_dim;
    printf("%s\n", kvd_version());

    uint8_t* k_host = (uint8_t*)read_file(dir, "k.bin", layer_bytes * n_layers);
    uint8_t* v_host = (uint8_t*)read_file(dir, "v.bin", layer_bytes * n_layers);
    float* q_host = (float*)read_file(dir, "q.bin", q_floats * sizeof(float) * n_layers);

    HIP_OK(hipSetDevice(0));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    void* ws = NULL;
    size_t ws_bytes = 0;
    float* q_dev;
    float* out_dev;
    HIP_OK(hipMalloc((void**)&q_dev, q_floats * sizeof(float) * n_layers));
    HIP_OK(hipMalloc((void**)&out_dev, q_floats * sizeof(float) * n_layers));
    HIP_OK(hipMemcpy(q_dev, q_host, q_floats * sizeof(float) * n_layers, hipMemcpyHostToDevice));
    float* out_host = (float*)malloc(q_floats * sizeof(float) * n_layers);

    /* 1. device-resident layer 0 */
    void* k_dev;
    void* v_dev;
    HIP_OK(hipMalloc(&k_dev, layer_bytes));
    HIP_OK(hipMalloc(&v_dev, layer_bytes));
    HIP_OK(hipMemcpy(k_dev, k_host, layer_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v_dev, v_host, layer_bytes, hipMemcpyHostToDevice));
    attend(q_dev, out_dev, k_dev, v_dev, n_rows, row_bytes, n_head_q, n_head_kv, head_dim, &ws, &ws_bytes, s);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(out_host, out_dev, q_floats * sizeof(float), hipMemcpyDeviceToHost));
    write_file(dir, "out_device.bin", out_host, q_floats * sizeof(float));

    /* 2. host-resident stack through the ring, depth 0 and depth 1 */
    uint8_t* kp;
    uint8_t* vp;
    HIP_OK(hipHostMalloc((void**)&kp, layer_bytes * n_layers, hipHostMallocDefault));
    HIP_OK(hipHostMalloc((void**)&vp, layer_bytes * n_layers, hipHostMallocDefault));
    memcpy(kp, k_host, layer_bytes * n_layers);
    memcpy(vp, v_host, layer_bytes * n_layers);
    void* ordered_k;
    void* ordered_v;
    HIP_OK(hipMalloc(&ordered_k, layer_bytes));
    HIP_OK(hipMalloc(&ordered_v, layer_bytes));
    for (int depth = 0; depth <= 1; ++depth) {
        kvd_ring* ring = kvd_ring_create(depth, (size_t)1 << 30);
        if (!ring) {
            fprintf(stderr, "kvd_ring_create: %s\n", kvd_last_error());
            return 3;
        }
        for (int step = 0; step < 2; ++step) {
            for (int l = 0; l < n_layers; ++l) {
                kvd_stage_args st;
                memset(&st, 0, sizeof st);
                st.layer = l;
                st.flags = KVD_STAGE_ACQUIRE;
                st.host_k = kp + (size_t)l * layer_bytes;
                st.host_v = vp + (size_t)l * layer_bytes;
                st.row_bytes = row_bytes;
                st.n_rows = n_rows;
                st.stable_rows = n_rows - 1;
                st.cap_rows = n_rows;
                st.ordered_k = ordered_k;
                st.ordered_v = ordered_v;
                kvd_slot_view view;
                KVD_OK_OR_DIE(kvd_ring_stage_layer(ring, &st, s, &view));
                attend(q_dev + (size_t)l * q_floats, out_dev + (size_t)l * q_floats, view.k, view.v, view.n_rows,
                       view.row_stride, n_head_q, n_head_kv, head_dim, &ws, &ws_bytes, s);
                KVD_OK_OR_DIE(kvd_ring_release(ring, l, s));
                if (depth > 0 && l + depth < n_layers) {
                    kvd_stage_args pf = st;
                    pf.layer = l + depth;
                    pf.flags = KVD_STAGE_PREFETCH;
                    pf.host_k = kp + (size_t)(l + depth) * layer_bytes;
                    pf.host_v = vp + (size_t)(l + depth) * layer_bytes;
                    KVD_OK_OR_DIE(kvd_ring_stage_layer(ring, &pf, s, NULL));
                }
            }
            HIP_OK(hipStreamSynchronize(s));
        }
        HIP_OK(hipMemcpy(out_host, out_dev, q_floats * sizeof(float) * n_layers, hipMemcpyDeviceToHost));
        write_file(dir, depth ? "out_ring_d1.bin" : "out_ring_d0.bin", out_host, q_floats * sizeof(float) * n_layers);
        kvd_ring_stats stats;
        KVD_OK_OR_DIE(kvd_ring_stats_get(ring, &stats, sizeof stats));
        printf("depth %d: engaged %d ring_bytes %lld n_prefetch %lld pipelined %lld primed %lld ordered %lld\n", depth,
               stats.engaged, (long long)stats.ring_bytes, (long long)stats.n_prefetch,
               (long long)stats.n_acquire_pipelined, (long long)stats.n_acquire_primed,
               (long long)stats.n_acquire_ordered);
        kvd_ring_destroy(ring);
    }

    /* 3. an invalid call is refused before anything is enqueued */
    {
        kvd_attn_args a;
        memset(&a, 0, sizeof a);
        a.n_seq = 1;
        a.n_head_q = n_head_q;
        a.n_head_kv = n_head_kv;
        a.head_dim = 96;
        int r = kvd_attend_decode(&a, s);
        printf("invalid head_dim -> %d (%s)\n", r, kvd_last_error());
        if (r != KVD_EINVAL || kvd_last_error()[0] == 0) return 5;
    }

    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipFree(ordered_k));
    HIP_OK(hipFree(ordered_v));
    HIP_OK(hipHostFree(kp));
    HIP_OK(hipHostFree(vp));
    HIP_OK(hipFree(k_dev));
    HIP_OK(hipFree(v_dev));
    HIP_OK(hipFree(q_dev));
    HIP_OK(hipFree(out_dev));
    if (ws) HIP_OK(hipFree(ws));
    HIP_OK(hipStreamDestroy(s));
    free(k_host);
    free(v_host);
    free(q_host);
    free(out_host);
    printf("ok\n");
    return 0;
}
