// lce_kernels.hip -- the kernels of the linear + cross-entropy path around
// the library GEMMs: per-chunk row statistics, the combine into the loss,
// and the bf16 gradient chunk.  Row arithmetic as in ce_device.h.
#include "ce_device.h"
#include "lce_internal.h"

namespace lce {
namespace {

using namespace cek;

constexpr float kNegInf = -__builtin_inff();

// Elements of fp32 vector v (columns 4v .. 4v+3 of the chunk) at or past vn,
// and the target's column tl, replaced with -inf.
__device__ __forceinline__ Vec mask_chunk(Vec x, int v, int vn, int tl)
{
    if (4 * v + 4 > vn)
        mask_outside<DT_F32>(x, 0, vn - 4 * v);
    if (tl >= 0 && tl / 4 == v)
        set_elem<DT_F32>(x, tl & 3, kNegInf);
    return x;
}

// (max, sum of exp(x - max)) of each row of the chunk with the target column
// left out, and the target's logit when the chunk holds it.
__global__ void __launch_bounds__(256) stats_kernel(LceParams q)
{
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= q.M)
        return;
    const Vec *x = reinterpret_cast<const Vec *>(q.L + row * q.ldc);
    const int64_t t = q.targets[row] - q.v0;
    const int tl = (t >= 0 && t < q.vn) ? (int)t : -1;
    const int nvec = (q.vn + 3) / 4;
    float m_run = kNegInf;
    float s_run = 0.0f;
    for (int base = 0; base < nvec; base += 64 * U) {
        Vec r[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int v = base + lane + 64 * k;
            r[k] = ldv(&x[v < nvec ? v : nvec - 1]);
        }
        float cm = m_run;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int v = base + lane + 64 * k;
            r[k] = mask_chunk(r[k], v, q.vn, tl);
            cm = v < nvec ? vec_max<DT_F32>(r[k], cm) : cm;
        }
        if (cm != kNegInf) {
            const float cmL = cm * kLog2e;
            float add = 0.0f;
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const float e = vec_sumexp<DT_F32>(r[k], cmL);
                add += (base + lane + 64 * k) < nvec ? e : 0.0f;
            }
            s_run = rescale_to(s_run, m_run, cm) + add;
            m_run = cm;
        }
    }
    const float m = group_reduce<64>(m_run, OpMax());
    const float s = group_reduce<64>(rescale_to(s_run, m_run, m), OpSum());
    if (lane == 0) {
        float *st = q.stats + 2 * (row * q.nchunks + q.chunk_index);
        st[0] = m;
        st[1] = s;
        if (tl >= 0)
            q.rowx[row] = q.L[row * q.ldc + tl];
    }
}

// The row's loss, lse and target gradient from its chunks' statistics
// (combined in chunk order per lane, then across lanes in a fixed tree).
__global__ void __launch_bounds__(256) finish_kernel(LceParams q)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= q.M)
        return;
    const float *st = q.stats + 2 * row * q.nchunks;
    float mi = kNegInf;
    float si = 0.0f;
    for (int c = lane; c < q.nchunks; c += 64) {
        const float m2 = st[2 * c];
        const float s2 = st[2 * c + 1];
        const float mn = fmaxf(mi, m2);
        si = rescale_to(si, mi, mn) + rescale_to(s2, m2, mn);
        mi = mn;
    }
    const float m_ex = group_reduce<64>(mi, OpMax());
    const float s_ex = group_reduce<64>(rescale_to(si, mi, m_ex), OpSum());
    const int64_t t = q.targets[row];
    const bool valid = (uint64_t)t < (uint64_t)q.V;
    const float xt = valid ? q.rowx[row] : __builtin_nanf("");
    const float m = valid ? fmaxf(m_ex, xt) : m_ex;
    const float mL = m * kLog2e;
    const float s_excl = rescale_to(s_ex, m_ex, m);
    const float et = valid ? fast_exp2(__builtin_fmaf(xt, kLog2e, -mL)) : 0.0f;
    const float s = s_excl + et;
    const bool accurate = valid && et > 0.5f * s;
    const RowResult rr = row_result(valid, m, xt, et, s, s_excl, accurate, q.c);
    if (lane == 0) {
        const float lse = m + kLn2 * __log2f(s);
        q.lse[row] = lse;
        if (q.lse_out)
            q.lse_out[row] = lse;
        q.gt[row] = rr.gt;
        if (q.partials)
            q.partials[row] = (double)rr.loss;
        else if (q.out)
            q.out[row] = rr.loss;
    }
}

// G = exp(L - lse) c in bf16 (round to nearest even), the target's column
// taking the gradient the combine computed; columns past vn are 0.
__global__ void __launch_bounds__(256) grad_kernel(LceParams q)
{
    constexpr int U = 4;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= q.M)
        return;
    const Vec *x = reinterpret_cast<const Vec *>(q.L + row * q.ldc);
    Vec *g = reinterpret_cast<Vec *>(q.G + row * q.ldc);
    const int64_t t = q.targets[row] - q.v0;
    const int tl = (t >= 0 && t < q.vn) ? (int)t : -1;
    const float gt = q.gt[row];
    // exp(x - lse) c = 2^(x log2 e - (lse log2 e - log2 c)), c > 0
    const float bias = q.lse[row] * kLog2e - __log2f(q.c);
    const int nout = (q.vn + 7) / 8;   // 8 bf16 per 16-byte output vector
    for (int base = 0; base < nout; base += 64 * U) {
        Vec a[U], b[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int v = base + lane + 64 * k;
            const int vv = v < nout ? v : nout - 1;
            a[k] = ldv(&x[2 * vv]);
            b[k] = ldv(&x[2 * vv + 1]);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int v = base + lane + 64 * k;
            if (v >= nout)
                continue;
            float e[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e[j] = fast_exp2(__builtin_fmaf(__uint_as_float(a[k].w[j]), kLog2e, -bias));
                e[4 + j] = fast_exp2(__builtin_fmaf(__uint_as_float(b[k].w[j]), kLog2e, -bias));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = 8 * v + j;
                e[j] = col == tl ? gt : (col < q.vn ? e[j] : 0.0f);
            }
            Vec o;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o.w[j] = pack2<DT_BF16>(e[2 * j], e[2 * j + 1]);
            stv(&g[v], o);
        }
    }
}

__global__ void __launch_bounds__(256) zero_kernel(float *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0.0f;
}

}  // namespace

const void *stats_kernel_fn() { return (const void *)&stats_kernel; }
const void *finish_kernel_fn() { return (const void *)&finish_kernel; }
const void *grad_kernel_fn() { return (const void *)&grad_kernel; }
const void *zero_kernel_fn() { return (const void *)&zero_kernel; }

}  // namespace lce
