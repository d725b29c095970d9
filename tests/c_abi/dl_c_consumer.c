/*
 * A plain C consumer of the DeltaLog C ABI (include/deltalog.h): device memory
 * from hipMalloc, no Python, no torch.  Test infrastructure: the GPU test
 * writes a seeded fp32 workload into a directory, runs this program on it and
 * compares what it writes back with the fp64 oracle.
 *
 *   dl_c_consumer <dir>        decode on the GPU
 *   dl_c_consumer --dry        host-only pool: bookkeeping only, no GPU needed
 *
 * <dir>/desc.txt   "P B H_v H_k d L decay update steps value_tile replay_split [window]"
 *                  (window W > 0: the last W steps go through one dl_decode_window call;
 *                  every step must then decode the same slots)
 * <dir>/init.bin   fp32 [P, H_v, d, d] initial states (natural layout)
 * <dir>/ids.bin    int32 [steps, B] slot ids per step
 * <dir>/q.bin, k.bin  fp32 [steps, B, H_k, d];  v.bin fp32 [steps, B, H_v, d]
 * <dir>/lam.bin    fp32 [steps, B, H_v] (scalar) or [steps, B, H_v, d] (per key); absent for no decay
 * <dir>/beta.bin   fp32 [steps, B, H_v]; absent for plain updates
 * Writes out.bin (fp32 [steps, B, H_v, d]), state.bin (fp32 [P, H_v, d, d],
 * after dl_flush_all) and loglen.txt (host mirror of the live lengths before
 * the flush, then the device counters' sum after it).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "deltalog.h"

#define CHECK_DL(call)                                                                   \
    do {                                                                                 \
        int rc_ = (call);                                                                \
        if (rc_ != DL_OK) {                                                              \
            fprintf(stderr, "%s failed (%d): %s\n", #call, rc_, dl_last_error());        \
            exit(2);                                                                     \
        }                                                                                \
    } while (0)
#define CHECK_HIP(call)                                                                  \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
            exit(3);                                                                     \
        }                                                                                \
    } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes, int required) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        if (required) {
            fprintf(stderr, "missing %s\n", path);
            exit(4);
        }
        return NULL;
    }
    void *buf = malloc(bytes ? bytes : 1);
    if (!buf || fread(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "short read of %s (%zu bytes expected)\n", path, bytes);
        exit(4);
    }
    fclose(f);
    return buf;
}

static void write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(5);
    }
    fclose(f);
}

static void *dev_copy(const void *host, size_t bytes) {
    void *d = NULL;
    if (!host) return NULL;
    CHECK_HIP(hipMalloc(&d, bytes));
    CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* Host-only pool: the append/merge schedule of 3 slots at L = 4 over a fixed
 * call sequence, printed as the live lengths after each call. */
static int dry_run(void) {
    dl_pool_desc d;
    memset(&d, 0, sizeof d);
    d.num_slots = 3;
    d.max_batch = 3;
    d.num_v_heads = 2;
    d.num_k_heads = 1;
    d.d_k = d.d_v = 64;
    d.merge_interval = 4;
    d.decay = DL_DECAY_SCALAR;
    d.update = DL_UPDATE_DELTA;
    d.state_dtype = DL_F32;
    d.in_dtype = DL_F32;
    dl_pool *pool = NULL;
    CHECK_DL(dl_pool_create(&d, NULL, &pool));
    const int32_t all[3] = {0, 1, 2}, two[2] = {2, 0}, dup[2] = {1, 1};
    int32_t n[3];
    for (int t = 0; t < 6; ++t) {
        if (t == 2) CHECK_DL(dl_merge(pool, 1, two, NULL));
        CHECK_DL(dl_decode_step(pool, t % 2 ? 2 : 3, t % 2 ? two : all, NULL, NULL, NULL, NULL, NULL, NULL, NULL));
        CHECK_DL(dl_get_log_len(pool, n));
        printf("%d %d %d\n", n[0], n[1], n[2]);
    }
    /* a refused call leaves the mirror alone */
    if (dl_decode_step(pool, 2, dup, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != DL_ERR_DUPLICATE_SLOT) return 6;
    CHECK_DL(dl_get_log_len(pool, n));
    printf("%d %d %d\n", n[0], n[1], n[2]);
    CHECK_DL(dl_pool_destroy(pool));
    return 0;
}

int main(int argc, char **argv) {
    if (argc == 2 && strcmp(argv[1], "--dry") == 0) return dry_run();
    if (argc != 2) {
        fprintf(stderr, "usage: %s <dir> | --dry\n", argv[0]);
        return 1;
    }
    const char *dir = argv[1];
    int P, B, Hv, Hk, D, L, decay, update, steps, value_tile, split, window = 0;
    {
        char path[4096];
        snprintf(path, sizeof path, "%s/desc.txt", dir);
        FILE *f = fopen(path, "r");
        if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d", &P, &B, &Hv, &Hk, &D, &L, &decay, &update, &steps,
                         &value_tile, &split) != 11) {
            fprintf(stderr, "bad %s\n", path);
            return 4;
        }
        if (fscanf(f, "%d", &window) != 1) window = 0;
        fclose(f);
        if (window < 0 || window > steps) {
            fprintf(stderr, "window %d outside [0, %d]\n", window, steps);
            return 4;
        }
    }
    dl_pool_desc d;
    memset(&d, 0, sizeof d);
    d.num_slots = P;
    d.max_batch = B;
    d.num_v_heads = Hv;
    d.num_k_heads = Hk;
    d.d_k = d.d_v = D;
    d.merge_interval = L;
    d.decay = decay;
    d.update = update;
    d.state_dtype = DL_F32;
    d.in_dtype = DL_F32;
    d.value_tile = value_tile;
    d.replay_split = split;

    /* pool buffers: the sizes the library asks for, from hipMalloc */
    size_t sz[DL_NUM_BUFS];
    CHECK_DL(dl_pool_sizes(&d, sz));
    void *bufp[DL_NUM_BUFS];
    for (int i = 0; i < DL_NUM_BUFS; ++i) {
        bufp[i] = NULL;
        if (sz[i]) CHECK_HIP(hipMalloc(&bufp[i], sz[i]));
    }
    dl_pool_buffers bufs = {bufp[DL_BUF_BASE], bufp[DL_BUF_KLOG], bufp[DL_BUF_ULOG], (float *)bufp[DL_BUF_LAMLOG],
                            (int32_t *)bufp[DL_BUF_NLOG], (float *)bufp[DL_BUF_COEF]};
    dl_pool *pool = NULL;
    CHECK_DL(dl_pool_create(&d, &bufs, &pool));

    const size_t head = (size_t)D * D, lam_w = decay == DL_DECAY_PER_KEY ? (size_t)D : 1;
    float *init = (float *)read_file(dir, "init.bin", (size_t)P * Hv * head * 4, 1);
    int32_t *ids = (int32_t *)read_file(dir, "ids.bin", (size_t)steps * B * 4, 1);
    float *q = (float *)read_file(dir, "q.bin", (size_t)steps * B * Hk * D * 4, 1);
    float *k = (float *)read_file(dir, "k.bin", (size_t)steps * B * Hk * D * 4, 1);
    float *v = (float *)read_file(dir, "v.bin", (size_t)steps * B * Hv * D * 4, 1);
    float *lam = decay == DL_DECAY_NONE ? NULL
                                        : (float *)read_file(dir, "lam.bin", (size_t)steps * B * Hv * lam_w * 4, 1);
    float *beta = update == DL_UPDATE_DELTA ? (float *)read_file(dir, "beta.bin", (size_t)steps * B * Hv * 4, 1)
                                            : NULL;

    /* initial states, in the natural layout, slots 0 .. P-1 */
    float *d_init = (float *)dev_copy(init, (size_t)P * Hv * head * 4);
    int32_t *all = (int32_t *)malloc((size_t)P * 4);
    for (int s = 0; s < P; ++s) all[s] = s;
    for (int lo = 0; lo < P; lo += B) {
        const int cnt = P - lo < B ? P - lo : B;
        CHECK_DL(dl_slot_assign(pool, cnt, all + lo, d_init + (size_t)lo * Hv * head, NULL));
    }

    float *d_q = (float *)dev_copy(q, (size_t)steps * B * Hk * D * 4);
    float *d_k = (float *)dev_copy(k, (size_t)steps * B * Hk * D * 4);
    float *d_v = (float *)dev_copy(v, (size_t)steps * B * Hv * D * 4);
    float *d_lam = (float *)dev_copy(lam, (size_t)steps * B * Hv * lam_w * 4);
    float *d_beta = (float *)dev_copy(beta, (size_t)steps * B * Hv * 4);
    float *d_out = NULL;
    CHECK_HIP(hipMalloc((void **)&d_out, (size_t)steps * B * Hv * D * 4));
    const int nstep = steps - window;
    for (int t = 0; t < nstep; ++t) {
        CHECK_DL(dl_decode_step(pool, B, ids + (size_t)t * B, d_q + (size_t)t * B * Hk * D, d_k + (size_t)t * B * Hk * D,
                                d_v + (size_t)t * B * Hv * D, d_lam ? d_lam + (size_t)t * B * Hv * lam_w : NULL,
                                d_beta ? d_beta + (size_t)t * B * Hv : NULL, d_out + (size_t)t * B * Hv * D, NULL));
    }
    if (window > 0) {   /* the remaining steps' inputs and outputs are contiguous, step-major */
        const size_t t = (size_t)nstep;
        CHECK_DL(dl_decode_window(pool, B, ids + t * B, window, d_q + t * B * Hk * D, d_k + t * B * Hk * D,
                                  d_v + t * B * Hv * D, d_lam ? d_lam + t * B * Hv * lam_w : NULL,
                                  d_beta ? d_beta + t * B * Hv : NULL, d_out + t * B * Hv * D, NULL));
    }
    int32_t *n = (int32_t *)malloc((size_t)P * 4);
    CHECK_DL(dl_get_log_len(pool, n));
    CHECK_DL(dl_flush_all(pool, NULL));

    float *d_state = NULL;
    CHECK_HIP(hipMalloc((void **)&d_state, (size_t)P * Hv * head * 4));
    for (int lo = 0; lo < P; lo += B) {
        const int cnt = P - lo < B ? P - lo : B;
        CHECK_DL(dl_read_base(pool, cnt, all + lo, d_state + (size_t)lo * Hv * head, NULL));
    }
    const int nv = D / dl_value_tile(&d);
    int32_t *dev_n = (int32_t *)malloc((size_t)P * Hv * nv * 4);
    CHECK_DL(dl_read_log_len_device(pool, dev_n, NULL));
    CHECK_HIP(hipDeviceSynchronize());

    float *out = (float *)malloc((size_t)steps * B * Hv * D * 4);
    float *state = (float *)malloc((size_t)P * Hv * head * 4);
    CHECK_HIP(hipMemcpy(out, d_out, (size_t)steps * B * Hv * D * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(state, d_state, (size_t)P * Hv * head * 4, hipMemcpyDeviceToHost));
    write_file(dir, "out.bin", out, (size_t)steps * B * Hv * D * 4);
    write_file(dir, "state.bin", state, (size_t)P * Hv * head * 4);
    {
        char path[4096];
        snprintf(path, sizeof path, "%s/loglen.txt", dir);
        FILE *f = fopen(path, "w");
        long sum = 0;
        for (int i = 0; i < P * Hv * nv; ++i) sum += dev_n[i];
        for (int s = 0; s < P; ++s) fprintf(f, "%d ", n[s]);
        fprintf(f, "\n%ld\n", sum);
        fclose(f);
    }

    CHECK_DL(dl_pool_destroy(pool));
    for (int i = 0; i < DL_NUM_BUFS; ++i)
        if (bufp[i]) CHECK_HIP(hipFree(bufp[i]));
    hipFree(d_init);
    hipFree(d_q);
    hipFree(d_k);
    hipFree(d_v);
    if (d_lam) hipFree(d_lam);
    if (d_beta) hipFree(d_beta);
    hipFree(d_out);
    hipFree(d_state);
    free(init); free(ids); free(q); free(k); free(v); free(lam); free(beta);
    free(all); free(n); free(dev_n); free(out); free(state);
    printf("ok\n");
    return 0;
}
