/*
 * ce_consumer.c -- a plain C99 program that drives the library through its C
 * ABI alone: no Python, no torch; device memory from hipMalloc, a stream of
 * its own, the headers included as C.  Test infrastructure: the GPU test
 * runs it and checks what it wrote against the fp64 oracle.
 *
 * usage: ce_consumer OUTDIR DTYPE M V SEED
 *   DTYPE 0 fp32, 1 fp16, 2 bf16.
 *
 * Inputs (seeded, synthetic): logits n/16 with n uniform in [-128, 128)
 * (exact in all three storage types), about 1 in 200 entries -inf (never at
 * the target), targets uniform in [0, V).  The logits start one element
 * past a 256-byte boundary, so rows are not 16-byte aligned.
 *
 * Calls, in order, on one stream with one workspace: ce_fwd (none, mean),
 * ce_fwd_lse (sum), ce_bwd from that lse (mean), ce_softmax and its log
 * form, ce_fwd_bwd_inplace (mean) on a copy of the logits, then ce_linear_fwd
 * (mean) on small bf16 H [64, 96] and W [1000, 96]; and four calls that must
 * fail before any launch (workspace too small, M < 0, unknown dtype, an
 * output at another 16-byte phase than the logits).  Every input and output
 * is written to OUTDIR as raw little-endian arrays; "ok" ends a clean run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ce.h"
#include "ce_linear.h"

static const char *g_dir;

#define HIP_CHECK(call)                                                          \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,          \
                    hipGetErrorString(e_));                                      \
            exit(2);                                                             \
        }                                                                        \
    } while (0)

#define CE_CHECK(call)                                                           \
    do {                                                                         \
        int s_ = (call);                                                         \
        if (s_ != CE_OK) {                                                       \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,          \
                    ce_status_string(s_));                                       \
            exit(3);                                                             \
        }                                                                        \
    } while (0)

#define CE_EXPECT(call, code)                                                    \
    do {                                                                         \
        int s_ = (call);                                                         \
        if (s_ != (code)) {                                                      \
            fprintf(stderr, "%s:%d %s returned %d (%s), expected %s\n", __FILE__, \
                    __LINE__, #call, s_, ce_status_string(s_), #code);           \
            exit(4);                                                             \
        }                                                                        \
    } while (0)

/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014) */
static uint64_t g_state;
static uint64_t next_u64(void)
{
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* uniform in [0, n) (the modulo bias is irrelevant here) */
static int64_t below(int64_t n) { return (int64_t)(next_u64() % (uint64_t)n); }

/* n / 16 in each storage format, for -128 <= n < 128 */
static uint32_t f32_bits(int n)
{
    float f = (float)n / 16.0f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static uint16_t bf16_bits(int n) { return (uint16_t)(f32_bits(n) >> 16); }

static uint16_t f16_bits(int n)
{
    if (n == 0)
        return 0;
    uint16_t sign = n < 0 ? 0x8000u : 0u;
    unsigned a = (unsigned)(n < 0 ? -n : n);
    int e = 0;
    while ((a >> (e + 1)) != 0)
        ++e;                                        /* 2^e <= a < 2^(e+1) */
    /* a / 16 = (a / 2^e) 2^(e - 4): biased exponent e - 4 + 15, and the
     * 10-bit fraction (a / 2^e - 1) 2^10, exact since a has e + 1 <= 8 bits */
    uint16_t frac = (uint16_t)(((a << 10) >> e) - 1024u);
    return (uint16_t)(sign | (uint16_t)((e - 4 + 15) << 10) | frac);
}

static void save(const char *name, const void *p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(5);
    }
    fclose(f);
}

/* copies n bytes of device memory to a fresh host buffer and saves it */
static void save_device(const char *name, const void *d, size_t n)
{
    void *h = malloc(n ? n : 1);
    if (!h)
        exit(6);
    HIP_CHECK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
    save(name, h, n);
    free(h);
}

int main(int argc, char **argv)
{
    if (argc != 6) {
        fprintf(stderr, "usage: %s OUTDIR DTYPE M V SEED\n", argv[0]);
        return 1;
    }
    g_dir = argv[1];
    const ce_dtype_t dt = (ce_dtype_t)atoi(argv[2]);
    const int64_t M = atoll(argv[3]), V = atoll(argv[4]);
    g_state = (uint64_t)atoll(argv[5]);
    if (dt < CE_F32 || dt > CE_BF16 || M < 1 || V < 2) {
        fprintf(stderr, "bad arguments\n");
        return 1;
    }
    const size_t es = dt == CE_F32 ? 4 : 2;
    const size_t nx = (size_t)M * (size_t)V * es;

    /* host inputs */
    uint8_t *hx = malloc(nx);
    int64_t *ht = malloc((size_t)M * sizeof(int64_t));
    if (!hx || !ht)
        return 6;
    for (int64_t i = 0; i < M; ++i)
        ht[i] = below(V);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < V; ++j) {
            const size_t o = (size_t)i * (size_t)V + (size_t)j;
            const int n = (int)below(256) - 128;
            const int ninf = j != ht[i] && below(200) == 0;
            if (dt == CE_F32) {
                uint32_t u = ninf ? 0xff800000u : f32_bits(n);
                memcpy(hx + 4 * o, &u, 4);
            } else {
                uint16_t u = ninf ? (dt == CE_F16 ? 0xfc00u : 0xff80u)
                                  : (dt == CE_F16 ? f16_bits(n) : bf16_bits(n));
                memcpy(hx + 2 * o, &u, 2);
            }
        }
    save("x.bin", hx, nx);
    save("t.bin", ht, (size_t)M * sizeof(int64_t));

    /* device buffers: every [M, V] one element past a 256-byte boundary */
    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    uint8_t *dx0, *dg0, *ds0, *dl0, *dxg0;
    HIP_CHECK(hipMalloc((void **)&dx0, nx + 256));
    HIP_CHECK(hipMalloc((void **)&dg0, nx + 256));
    HIP_CHECK(hipMalloc((void **)&ds0, nx + 256));
    HIP_CHECK(hipMalloc((void **)&dl0, nx + 256));
    HIP_CHECK(hipMalloc((void **)&dxg0, nx + 256));
    uint8_t *dx = dx0 + es, *dg = dg0 + es, *ds = ds0 + es, *dl = dl0 + es, *dxg = dxg0 + es;
    int64_t *dt_ = NULL;
    float *loss_none, *loss_mean, *loss_sum, *lse, *loss_fused;
    HIP_CHECK(hipMalloc((void **)&dt_, (size_t)M * sizeof(int64_t)));
    HIP_CHECK(hipMalloc((void **)&loss_none, (size_t)M * sizeof(float)));
    HIP_CHECK(hipMalloc((void **)&lse, (size_t)M * sizeof(float)));
    HIP_CHECK(hipMalloc((void **)&loss_mean, sizeof(float)));
    HIP_CHECK(hipMalloc((void **)&loss_sum, sizeof(float)));
    HIP_CHECK(hipMalloc((void **)&loss_fused, sizeof(float)));
    const size_t wsb = ce_workspace_bytes(M, V, dt, CE_MEAN);
    void *ws = NULL;
    HIP_CHECK(hipMalloc(&ws, wsb));
    HIP_CHECK(hipMemcpy(dx, hx, nx, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dt_, ht, (size_t)M * sizeof(int64_t), hipMemcpyHostToDevice));

    char plan[256];
    CE_CHECK(ce_plan_describe(M, V, dt, CE_MEAN, CE_OP_FWD, plan, sizeof plan));
    printf("M %lld V %lld dtype %d workspace %zu plan %s\n", (long long)M, (long long)V,
           (int)dt, wsb, plan);

    CE_CHECK(ce_fwd(dx, dt_, M, V, dt, CE_NONE, loss_none, NULL, 0, stream));
    CE_CHECK(ce_fwd(dx, dt_, M, V, dt, CE_MEAN, loss_mean, ws, wsb, stream));
    CE_CHECK(ce_fwd_lse(dx, dt_, M, V, dt, CE_SUM, loss_sum, lse, ws, wsb, stream));
    CE_CHECK(ce_bwd(dx, dt_, lse, NULL, M, V, dt, CE_MEAN, dg, ws, wsb, stream));
    CE_CHECK(ce_softmax(dx, M, V, dt, 0, ds, NULL, ws, wsb, stream));
    CE_CHECK(ce_softmax(dx, M, V, dt, 1, dl, NULL, ws, wsb, stream));
    HIP_CHECK(hipMemcpyAsync(dxg, dx, nx, hipMemcpyDeviceToDevice, stream));
    CE_CHECK(ce_fwd_bwd_inplace(dxg, dt_, M, V, dt, CE_MEAN, loss_fused, ws, wsb, stream));

    /* calls that must fail before any launch */
    CE_EXPECT(ce_fwd(dx, dt_, M, V, dt, CE_MEAN, loss_mean, ws, 1, stream), CE_ERR_WORKSPACE);
    CE_EXPECT(ce_fwd(dx, dt_, -1, V, dt, CE_NONE, loss_none, NULL, 0, stream), CE_ERR_SHAPE);
    CE_EXPECT(ce_fwd(dx, dt_, M, V, (ce_dtype_t)7, CE_NONE, loss_none, NULL, 0, stream),
              CE_ERR_DTYPE);
    CE_EXPECT(ce_softmax(dx, M, V, dt, 0, ds + es, NULL, NULL, 0, stream), CE_ERR_ALIGNMENT);
    HIP_CHECK(hipStreamSynchronize(stream));

    save_device("loss_none.bin", loss_none, (size_t)M * sizeof(float));
    save_device("loss_mean.bin", loss_mean, sizeof(float));
    save_device("loss_sum.bin", loss_sum, sizeof(float));
    save_device("lse.bin", lse, (size_t)M * sizeof(float));
    save_device("grad.bin", dg, nx);
    save_device("softmax.bin", ds, nx);
    save_device("log_softmax.bin", dl, nx);
    save_device("grad_fused.bin", dxg, nx);
    save_device("loss_fused.bin", loss_fused, sizeof(float));

    /* linear + cross-entropy on bf16 H [LM, LD], W [LV, LD] */
    enum { LM = 64, LD = 96, LV = 1000 };
    uint16_t *hh = malloc(sizeof(uint16_t) * LM * LD), *hw = malloc(sizeof(uint16_t) * LV * LD);
    int64_t *hlt = malloc(sizeof(int64_t) * LM);
    if (!hh || !hw || !hlt)
        return 6;
    for (int i = 0; i < LM * LD; ++i)
        hh[i] = bf16_bits((int)below(32) - 16);
    for (int i = 0; i < LV * LD; ++i)
        hw[i] = bf16_bits((int)below(32) - 16);
    for (int i = 0; i < LM; ++i)
        hlt[i] = below(LV);
    save("linear_h.bin", hh, sizeof(uint16_t) * LM * LD);
    save("linear_w.bin", hw, sizeof(uint16_t) * LV * LD);
    save("linear_t.bin", hlt, sizeof(int64_t) * LM);
    void *dh, *dw, *lws;
    int64_t *dlt;
    float *lin_loss, *lin_lse;
    const size_t lwsb = ce_linear_workspace_bytes(LM, LD, LV, 0);
    HIP_CHECK(hipMalloc(&dh, sizeof(uint16_t) * LM * LD));
    HIP_CHECK(hipMalloc(&dw, sizeof(uint16_t) * LV * LD));
    HIP_CHECK(hipMalloc((void **)&dlt, sizeof(int64_t) * LM));
    HIP_CHECK(hipMalloc((void **)&lin_loss, sizeof(float)));
    HIP_CHECK(hipMalloc((void **)&lin_lse, sizeof(float) * LM));
    HIP_CHECK(hipMalloc(&lws, lwsb));
    HIP_CHECK(hipMemcpy(dh, hh, sizeof(uint16_t) * LM * LD, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dw, hw, sizeof(uint16_t) * LV * LD, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dlt, hlt, sizeof(int64_t) * LM, hipMemcpyHostToDevice));
    CE_CHECK(ce_linear_fwd(dh, dw, dlt, LM, LD, LV, CE_MEAN, lin_loss, lin_lse, 0, lws, lwsb,
                           stream));
    HIP_CHECK(hipStreamSynchronize(stream));
    save_device("linear_loss.bin", lin_loss, sizeof(float));
    save_device("linear_lse.bin", lin_lse, sizeof(float) * LM);

    HIP_CHECK(hipFree(dx0));
    HIP_CHECK(hipFree(dg0));
    HIP_CHECK(hipFree(ds0));
    HIP_CHECK(hipFree(dl0));
    HIP_CHECK(hipFree(dxg0));
    HIP_CHECK(hipFree(dt_));
    HIP_CHECK(hipFree(loss_none));
    HIP_CHECK(hipFree(lse));
    HIP_CHECK(hipFree(loss_mean));
    HIP_CHECK(hipFree(loss_sum));
    HIP_CHECK(hipFree(loss_fused));
    HIP_CHECK(hipFree(ws));
    HIP_CHECK(hipFree(dh));
    HIP_CHECK(hipFree(dw));
    HIP_CHECK(hipFree(dlt));
    HIP_CHECK(hipFree(lin_loss));
    HIP_CHECK(hipFree(lin_lse));
    HIP_CHECK(hipFree(lws));
    HIP_CHECK(hipStreamDestroy(stream));
    free(hx);
    free(ht);
    free(hh);
    free(hw);
    free(hlt);
    printf("ok\n");
    return 0;
}
