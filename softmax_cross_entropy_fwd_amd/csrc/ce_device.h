// ce_device.h -- device code for row-wise softmax cross-entropy on gfx950.
//
// Internal to the library.  Three row mappings share the per-row arithmetic:
//
//   rows_kernel<G, K>   G lanes per row (64/G rows per wavefront), the whole
//                       row held in registers (K 16-byte vectors per lane).
//   wg_kernel<W, K>     one row per workgroup of W wavefronts, the whole row
//                       held in registers across the workgroup; cross-wave
//                       combine through LDS.
//   stream_kernel<W, K> one row per workgroup, streamed in chunks of
//                       W*64*K vectors with an online (max, sum) rescale; the
//                       backward re-reads the row.  Any row length.
//
// Per row (the cross-entropy of the POPCORNBENCH "Kimi-K2.6 l1_p95" trace and
// of loss_kernel in the Triton issue "Cross Entropy Loss performance issue"):
//   m   = max_j x_j
//   s   = sum_j 2^(x_j*log2e - m*log2e)          (fp32, exp2 on the VALU)
//   loss = (m - x_t) + ln 2 * log2(s)
// and, for the fused backward ("9 Triton kernels in 9 weeks", week 7),
//   g_j = 2^(x_j*log2e - m*log2e - log2(s)) * c,  g_t = (p_t - 1) * c,
// written over the row.  The two-phase form (row max first, then the sum
// against that max) replaces the pages' per-element online update wherever the
// row sits in registers; the chunked stream applies the pages' blockwise
// rescale once per chunk, in base 2 so it cannot overflow.
//
// When the target holds more than half of the probability mass (p_t > 1/2),
// 1 - p_t and the loss are recomputed from the sum of the other terms, so the
// target's gradient and a small loss keep their relative accuracy.
//
// Rows are read in aligned 16-byte vectors.  A row that does not start or end
// on a 16-byte boundary is covered by the aligned window around it; elements
// of the window outside the row are treated as -inf and never written.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cek {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum : int { RED_NONE = 0, RED_MEAN = 1, RED_SUM = 2 };
// What the kernels write over (or next to) the row once its log-sum-exp is
// known.  EPI_LSE_GRAD is the gradient from a log-sum-exp given per row (no
// reduction pass).
enum : int { EPI_NONE = 0, EPI_GRAD = 1, EPI_SOFTMAX = 2, EPI_LOGSOFTMAX = 3, EPI_LSE_GRAD = 4 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMaxPartials = 16384;   // units (wavefronts or workgroups) per grid

struct alignas(16) Vec {
    uint32_t w[4];
};

struct Params {
    Vec *x;                  // 16-byte aligned address at or before logits[0]
    const int64_t *targets;  // [M]
    float *out;              // [M] (none) or [1]
    double *partials;        // one loss sum per unit (wavefront or workgroup)
    int64_t M;
    int64_t V;
    int head0;               // elements between x and logits[0]
    int aligned;             // every row starts and ends on a 16-byte boundary
    int blocked;             // each workgroup takes a contiguous band of rows
    int reduction;
    float c;                 // gradient scale (1/M for mean, 1 otherwise)
    double out_scale;        // 1/M (mean) or 1 (sum)
    Vec *y;                  // epilogue output, same 16-byte phase as x (== x in place)
    const float *dloss;      // upstream gradient, [M] or [1] (see dloss_per_row); null means 1
    int dloss_per_row;       // dloss holds one value per row
    float *lse_out;          // optional [M] row log-sum-exps
    const float *lse_in;     // [M] given log-sum-exps (backward from saved statistics)
    // split rows: S workgroups per row, each over slice_vecs window vectors
    int S;
    int slice_vecs;
    float *stats;            // [M * S][2] slice (max, sum) with the target left out
    float *fix;              // [M * S] slice sums of p_j, j != t (backward from lse)
    float *rowx;             // [M] target logits, saved before any slice is overwritten
    // non-null (mean or sum over whole rows): the last workgroup to finish
    // adds the partials and writes out[0] in this launch (finish_in_kernel)
    unsigned *ticket;
};

// ------------------------------------------------------------ storage types

template <int DT> struct Traits;
template <> struct Traits<DT_F32> {
    static constexpr int E = 4;                  // elements per 16-byte vector
    static constexpr uint32_t kNegInfWord = 0xff800000u;
};
template <> struct Traits<DT_F16> {
    static constexpr int E = 8;
    static constexpr uint32_t kNegInfWord = 0xfc00fc00u;
};
template <> struct Traits<DT_BF16> {
    static constexpr int E = 8;
    static constexpr uint32_t kNegInfWord = 0xff80ff80u;
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// Element j (compile-time after unrolling) of a vector, widened to fp32.
template <int DT>
__device__ __forceinline__ float elem(const Vec &v, int j)
{
    if constexpr (DT == DT_F32) {
        return __uint_as_float(v.w[j]);
    } else if constexpr (DT == DT_BF16) {
        uint32_t w = v.w[j >> 1];
        return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        half2_t h = __builtin_bit_cast(half2_t, v.w[j >> 1]);
        return (float)((j & 1) ? h.y : h.x);
    }
}

// Replace the elements of v outside [lo, hi) with -inf.
template <int DT>
__device__ __forceinline__ void mask_outside(Vec &v, int lo, int hi)
{
    constexpr int E = Traits<DT>::E;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (j < lo || j >= hi) {
            if constexpr (DT == DT_F32) {
                v.w[j] = 0xff800000u;
            } else if constexpr (DT == DT_F16) {
                v.w[j >> 1] = (j & 1) ? ((v.w[j >> 1] & 0x0000ffffu) | 0xfc000000u)
                                      : ((v.w[j >> 1] & 0xffff0000u) | 0x0000fc00u);
            } else {
                v.w[j >> 1] = (j & 1) ? ((v.w[j >> 1] & 0x0000ffffu) | 0xff800000u)
                                      : ((v.w[j >> 1] & 0xffff0000u) | 0x0000ff80u);
            }
        }
    }
}

template <int DT>
__device__ __forceinline__ Vec neg_inf_vec()
{
    Vec v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v.w[i] = Traits<DT>::kNegInfWord;
    return v;
}

// Two fp32 gradients -> one 32-bit word of the storage type (RNE).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    if constexpr (DT == DT_BF16) {
        bf162_t r;
        r.x = (__bf16)a;
        r.y = (__bf16)b;
        return __builtin_bit_cast(uint32_t, r);
    } else {
        half2_t r;
        r.x = (_Float16)a;
        r.y = (_Float16)b;
        return __builtin_bit_cast(uint32_t, r);
    }
}

// Store elements [lo, hi) of v at p (a vector-aligned address) one by one.
template <int DT>
__device__ __forceinline__ void store_partial(Vec *p, const Vec &v, int lo, int hi)
{
    constexpr int E = Traits<DT>::E;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (j >= lo && j < hi) {
            if constexpr (DT == DT_F32) {
                reinterpret_cast<uint32_t *>(p)[j] = v.w[j];
            } else {
                uint32_t w = v.w[j >> 1];
                reinterpret_cast<uint16_t *>(p)[j] = (uint16_t)((j & 1) ? (w >> 16) : w);
            }
        }
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row data is read once and written once: loads and stores can carry the
// non-temporal (streaming) hint.  Stores do for rows that start and end on
// 16-byte boundaries (the outputs are not read again here); the rows of a
// misaligned batch share their boundary cache lines with their neighbours,
// and there plain stores, which let the cache merge the two rows' halves of a
// line, measured faster (stress rows' fused backward: 354 -> 335 us).  Loads
// do where nothing reads the row again and every load
// instruction of a wavefront covers whole 128-byte lines (NT): the forwards
// of rows of at least 8 lanes (measured on MI355X: 5-8 % faster for the
// classifier, LM-head and stress forwards).  The hint lets the line go
// early, so it is not used where the next load of the same line follows
// (rows of fewer than 8 lanes: 24 % slower for the skinny rows) or where the
// row is read again or written back in place (the epilogues: 6 % slower for
// the stress rows' fused backward).
template <bool NT = false>
__device__ __forceinline__ Vec ldv(const Vec *p)
{
    if constexpr (NT) {
        Vec v;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v.w[i] = __builtin_nontemporal_load(&p->w[i]);
        return v;
    } else {
        return *p;
    }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One 16-byte store.  Issued as a single vector store, so that the compiler
// cannot merge its words with the element-wise stores of a row's boundary
// vector (fp32 epilogues were split into 4- and 8-byte stores that way).
template <bool NT = true>
__device__ __forceinline__ void stv(Vec *p, const Vec &v)
{
    const u32x4_t x = {v.w[0], v.w[1], v.w[2], v.w[3]};
    if constexpr (NT)
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t *>(p));
    else
        *reinterpret_cast<u32x4_t *>(p) = x;
}

// A row's target read through the constant address space: the kernels never
// write the targets, and a uniform address then becomes a scalar load.  A
// vector load retires behind every row load already in flight, and the fused
// epilogues move the uniform value to a scalar register at once, which made
// them wait for all of them (vector loads complete in order).  (The given
// log-sum-exps and upstream gradients stay vector loads: read this way they
// measured 3-4 % slower in the backward from a given lse.)
template <class T>
__device__ __forceinline__ T row_scalar(const T *base, int64_t i)
{
    return ((const __attribute__((address_space(4))) T *)base)[i];
}

// ------------------------------------------------------- lane reductions
// DPP within 16-lane rows, a lane swap for 32, and readlane for 64.  Every
// lane of a G-lane group ends with the same (bitwise) result.

struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
    static constexpr float identity() { return -__builtin_inff(); }
};
struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
    static constexpr float identity() { return 0.0f; }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int G, class Op>
__device__ __forceinline__ float group_reduce(float v, Op op)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "G");
    if constexpr (G >= 2) v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v = op(v, dpp<0x141>(v));  // row_half_mirror
    if constexpr (G >= 16) v = op(v, dpp<0x140>(v)); // row_mirror
    if constexpr (G == 32) v = op(v, __shfl_xor(v, 16, 64));
    if constexpr (G == 64) {
        float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
        float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
        float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
        float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        v = op(op(a, b), op(c, d));
    }
    return v;
}

// Value of lane `src` of this lane's G-lane group.
template <int G>
__device__ __forceinline__ float group_bcast(float v, int src_in_group)
{
    if constexpr (G == 1) {
        return v;
    } else if constexpr (G == 64) {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_in_group));
    } else {
        int lane = threadIdx.x & 63;
        return __shfl(v, (lane & ~(G - 1)) + src_in_group, 64);
    }
}

// ------------------------------------------------------ per-row helpers

// Where the target sits in the row's window of vectors (32-bit: a window
// holds fewer than 2^31 elements).
struct TargetPos {
    bool valid;
    int vt;   // window vector index, -1 when the target is out of range
    int jt;   // element within the vector
};

template <int DT>
__device__ __forceinline__ TargetPos target_pos(int64_t t, int64_t V, int head)
{
    constexpr int E = Traits<DT>::E;
    TargetPos tp;
    tp.valid = (uint64_t)t < (uint64_t)V;
    const uint32_t wt = tp.valid ? (uint32_t)t + (uint32_t)head : 0u;
    tp.vt = tp.valid ? (int)(wt / E) : -1;
    tp.jt = (int)(wt % E);
    return tp;
}

// Keeps the compiler from carrying values derived from the row (widened
// elements, exponentials) from one pass to the next: each pass recomputes
// them from the packed registers, which bounds register use to the packed row.
template <int DT, int K>
__device__ __forceinline__ void opt_barrier(Vec (&raw)[K])
{
    if constexpr (DT != DT_F32) {   // fp32 elements need no widening
#pragma unroll
        for (int k = 0; k < K; ++k)
            asm volatile("" : "+v"(raw[k].w[0]), "+v"(raw[k].w[1]), "+v"(raw[k].w[2]),
                         "+v"(raw[k].w[3]));
    }
}

// Loads window vectors lidx + STRIDE*k (k < K) of a row whose window has nvec
// vectors and starts at xrow.  Every load is issued, in one block, before any
// is used: a lane whose vector lies past the window re-reads the window's last
// vector (a cache hit), and the caller drops that copy from the sum with
// vec_valid().  kfull (uniform) is the number of leading k for which every
// lane's vector lies inside every row's window.  Elements of the window
// outside the row become -inf; only the first and the last window vector (and
// copies of the last) can hold such elements.
// PART: vector slots that lie wholly past the window for this lane's
// wavefront (its first lane index is wfirst, wave-uniform) are not loaded and
// hold -inf.
template <int DT, int K, int STRIDE, bool NTL = false, bool PART = false>
__device__ __forceinline__ void load_window(Vec (&raw)[K], const Vec *xrow, int lidx, int nvec,
                                            int kfull, int head, int64_t V, bool aligned,
                                            int wfirst = 0)
{
    constexpr int E = Traits<DT>::E;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int v = lidx + STRIDE * k;
        if (!PART || wfirst + STRIDE * k < nvec)
            raw[k] = ldv<NTL>(&xrow[v < nvec ? v : nvec - 1]);
        else
            raw[k] = neg_inf_vec<DT>();
    }
    if (!aligned) {
        if (lidx == 0 && head > 0)
            mask_outside<DT>(raw[0], head, E);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (k + 1 >= kfull) {
                const int v = lidx + STRIDE * k;
                if (v >= nvec - 1)
                    mask_outside<DT>(raw[k], 0, (int)(head + V - (int64_t)(nvec - 1) * E));
            }
        }
    }
}

// Whether the lane's k-th vector is a window vector of its own (not a copy).
template <int STRIDE>
__device__ __forceinline__ bool vec_valid(int k, int kfull, int lidx, int nvec)
{
    return k < kfull || lidx + STRIDE * k < nvec;
}

// Per-row constants of the write epilogue, with p = 2^(x log2e - lse log2e):
//   GRAD        g = (p - [j == t]) * c      (the target's element is patched)
//   SOFTMAX     y = p
//   LOGSOFTMAX  y = x - lse
// log2|c| is folded into the exponent and the sign of c applied afterwards
// (c = 0 gives 0).  bf16, whose range reaches below fp32's normal range: the
// exponent is lifted by 64 and the product scaled by 2^-64, so results that
// round to bf16 subnormals are formed from normal fp32 values.  fp32: the
// exponent is (x - m) log2e - (log2 s - log2|c|), keeping it small and the
// relative error near 1e-6.
template <int DT>
struct EpiCoef {
    float m;
    float bias;
    float post;     // sign of c (and the 2^-64 lift for bf16)
    float lse;
};

template <int DT, int OP>
__device__ __forceinline__ EpiCoef<DT> epi_coef(float m, float mL, float log2s, float c)
{
    EpiCoef<DT> e;
    e.m = m;
    e.lse = m + kLn2 * log2s;
    const float ac = OP == EPI_GRAD ? fabsf(c) : 1.0f;
    const float sgn = (OP == EPI_GRAD && c < 0.0f) ? -1.0f : 1.0f;
    const float l2c = __log2f(ac);
    if constexpr (DT == DT_F32) {
        e.bias = log2s - l2c;
        e.post = sgn;
    } else if constexpr (DT == DT_F16) {
        e.bias = mL + log2s - l2c;
        e.post = sgn;
    } else {
        e.bias = mL + log2s - l2c - 64.0f;
        e.post = sgn * 5.42101086242752217e-20f;   // 2^-64
    }
    return e;
}

// The epilogue of one vector, packed to the storage type.
template <int DT, int OP>
__device__ __forceinline__ Vec epi_vec(const Vec &in, const EpiCoef<DT> &ec)
{
    constexpr int E = Traits<DT>::E;
    float g[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const float x = elem<DT>(in, j);
        if constexpr (OP == EPI_LOGSOFTMAX)
            g[j] = x - ec.lse;
        else if constexpr (DT == DT_F32)
            g[j] = fast_exp2(__builtin_fmaf(x - ec.m, kLog2e, -ec.bias)) * ec.post;
        else if constexpr (DT == DT_F16)
            g[j] = fast_exp2(__builtin_fmaf(x, kLog2e, -ec.bias));
        else
            g[j] = fast_exp2(__builtin_fmaf(x, kLog2e, -ec.bias)) * ec.post;
    }
    Vec out;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            out.w[j] = __float_as_uint(g[j]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            out.w[j] = pack2<DT>(g[2 * j], g[2 * j + 1]);
        if constexpr (DT == DT_F16 && OP != EPI_LOGSOFTMAX) {
            if (ec.post < 0.0f) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    out.w[j] ^= 0x80008000u;
            }
        }
    }
    return out;
}

template <int DT>
__device__ __forceinline__ float vec_max(const Vec &v, float m)
{
    constexpr int E = Traits<DT>::E;
#pragma unroll
    for (int j = 0; j < E; ++j)
        m = fmaxf(m, elem<DT>(v, j));
    return m;
}

// The same for fp16 on packed halves (max is exact in fp16, two elements per
// instruction).  Used where the widened elements are not needed right after
// (in the one-pass folds the widening is shared with the sum, and there the
// packed form measured slower).
__device__ __forceinline__ float vec_max_f16_packed(const Vec &v, float m)
{
    half2_t a = __builtin_bit_cast(half2_t, v.w[0]);
    half2_t b = __builtin_bit_cast(half2_t, v.w[1]);
    a = __builtin_elementwise_max(a, __builtin_bit_cast(half2_t, v.w[2]));
    b = __builtin_elementwise_max(b, __builtin_bit_cast(half2_t, v.w[3]));
    a = __builtin_elementwise_max(a, b);
    return fmaxf(m, fmaxf((float)a.x, (float)a.y));
}

// Sum of 2^(x*log2e - mL) over the vector (two chains for latency).
template <int DT>
__device__ __forceinline__ float vec_sumexp(const Vec &v, float mL)
{
    constexpr int E = Traits<DT>::E;
    float a = fast_exp2(__builtin_fmaf(elem<DT>(v, 0), kLog2e, -mL));
    float b = fast_exp2(__builtin_fmaf(elem<DT>(v, 1), kLog2e, -mL));
#pragma unroll
    for (int j = 2; j < E; j += 2) {
        a += fast_exp2(__builtin_fmaf(elem<DT>(v, j), kLog2e, -mL));
        b += fast_exp2(__builtin_fmaf(elem<DT>(v, j + 1), kLog2e, -mL));
    }
    return a + b;
}

// The same sum leaving out element jt.
template <int DT>
__device__ __forceinline__ float vec_sumexp_skip(const Vec &v, float mL, int jt)
{
    constexpr int E = Traits<DT>::E;
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        float e = fast_exp2(__builtin_fmaf(elem<DT>(v, j), kLog2e, -mL));
        a += (j == jt) ? 0.0f : e;
    }
    return a;
}

template <int DT>
__device__ __forceinline__ float vec_elem_dyn(const Vec &v, int jt)
{
    constexpr int E = Traits<DT>::E;
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j)
        if (j == jt)
            r = elem<DT>(v, j);
    return r;
}

// Loss and target gradient of a row from its reduced statistics.
struct RowResult {
    float loss;
    float gt;       // gradient of the target element (already times c)
};

__device__ __forceinline__ RowResult row_result(bool tvalid, float m, float xt, float et, float s,
                                                float s_excl, bool accurate, float c)
{
    RowResult r;
    if (!tvalid) {
        r.loss = __builtin_nanf("");
        r.gt = 0.0f;
        return r;
    }
    if (accurate) {
        r.loss = log1pf(s_excl / et);
        r.gt = -(s_excl / s) * c;
    } else {
        r.loss = (m - xt) + kLn2 * __log2f(s);
        r.gt = (et / s - 1.0f) * c;
    }
    return r;
}

// Writes window vector v of the epilogue output row, leaving elements outside
// the row untouched.
template <int DT>
__device__ __forceinline__ void store_grad(Vec *xrow, int v, const Vec &g, int head, int64_t V,
                                           bool aligned)
{
    constexpr int E = Traits<DT>::E;
    if (aligned) {
        stv(&xrow[v], g);
        return;
    }
    const int64_t lo = head - (int64_t)v * E;
    const int64_t hi = lo + V;
    if (lo <= 0 && hi >= E)
        stv<false>(&xrow[v], g);   // misaligned rows: plain stores (see stv)
    else
        store_partial<DT>(xrow + v, g, (int)(lo > 0 ? lo : 0), (int)(hi < E ? hi : E));
}

// ------------------------------------------- reductions across a row's lanes

// Combining per-lane online pairs (m, s) -- s being a sum of 2^((x - m) log2 e)
// -- into the row's (M, S): M = max m, S = sum s * 2^((m - M) log2 e).  A lane
// whose m equals M keeps its s exactly.
__device__ __forceinline__ float rescale_to(float s, float m, float M)
{
    return m == M ? s : s * fast_exp2((m - M) * kLog2e);
}

// G lanes of one wavefront per row.  share_xt: the target logit held by lane
// `owner_lane` of a row that spans the wavefront (G == 64 only).
template <int G>
struct GroupRed {
    __device__ __forceinline__ void combine(float m, float s, float &M, float &S)
    {
        M = group_reduce<G>(m, OpMax());
        S = group_reduce<G>(rescale_to(s, m, M), OpSum());
    }
    __device__ __forceinline__ float share_xt(float xt_own, int owner_lane)
    {
        static_assert(G == 64, "only a row spanning the wavefront has a uniform owner");
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xt_own),
                                                        __builtin_amdgcn_readfirstlane(owner_lane)));
    }
    __device__ __forceinline__ float sum_excl(float v) { return group_reduce<G>(v, OpSum()); }
    __device__ __forceinline__ void next_row() {}
};

// W wavefronts of one workgroup per row: DPP within each wavefront, LDS across
// them, partials combined in wavefront order, one barrier per row.  Slots
// alternate between two banks row by row: a wavefront can run at most one
// barrier ahead, so it never overwrites a bank another is still reading.
template <int W>
struct WgRed {
    float (*smax)[W];
    float (*ssum)[W];
    float (*sexc)[W];
    float *sxt;      // [2]: the target logit, written by its owner thread
    int wave, lane, bank;
    // owner: this thread holds the row's target logit xt_own; it is published
    // before the combine's barrier and read by everyone after it
    __device__ __forceinline__ void combine(float m, float s, float &M, float &S, float xt_own = 0.0f,
                                            bool owner = false)
    {
        const float mw = group_reduce<64>(m, OpMax());
        const float sw = group_reduce<64>(rescale_to(s, m, mw), OpSum());
        if (lane == 0) {
            smax[bank][wave] = mw;
            ssum[bank][wave] = sw;
        }
        if (owner)
            sxt[bank] = xt_own;
        __syncthreads();
        M = smax[bank][0];
#pragma unroll
        for (int w = 1; w < W; ++w)
            M = fmaxf(M, smax[bank][w]);
        S = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w)
            S += rescale_to(ssum[bank][w], smax[bank][w], M);
    }
    __device__ __forceinline__ float xt() const { return sxt[bank]; }
    __device__ __forceinline__ float sum_excl(float v)
    {
        v = group_reduce<64>(v, OpSum());
        if (lane == 0)
            sexc[bank][wave] = v;
        __syncthreads();
        float r = sexc[bank][0];
#pragma unroll
        for (int w = 1; w < W; ++w)
            r += sexc[bank][w];
        return r;
    }
    __device__ __forceinline__ void next_row() { bank ^= 1; }
};

// The logit x[row, t] read straight from memory (the row's own lines are being
// fetched at the same time, so this costs a cache hit), widened to fp32.
template <int DT>
__device__ __forceinline__ float load_logit(const Params &p, int64_t row, int64_t t)
{
    const int64_t e = row * p.V + p.head0 + t;
    if constexpr (DT == DT_F32) {
        return reinterpret_cast<const float *>(p.x)[e];
    } else {
        const uint16_t b = reinterpret_cast<const uint16_t *>(p.x)[e];
        if constexpr (DT == DT_BF16)
            return __uint_as_float((uint32_t)b << 16);
        else
            return (float)__builtin_bit_cast(_Float16, b);
    }
}

// Issues the loads of a row's window vectors lidx + STRIDE*k into raw.  EXACT:
// every row's window is exactly STRIDE*K vectors (aligned rows), so no index
// is clamped.  Otherwise a lane past the window re-reads the window's last
// vector (a cache hit) and the sums drop that copy (vec_valid).
// (The compiler may reorder these loads against the loop's refill order; its
// merged wait at the loop head then covers most of the row before the first
// vector is folded.  Kept in program order, the waits came per vector and the
// classifier forward ran 2-3 % slower, so the order is left to the compiler.)
template <int DT, int K, int STRIDE, bool EXACT, bool NTL = false>
__device__ __forceinline__ void issue_loads(Vec (&raw)[K], const Vec *xrow, int lidx, int nvec,
                                            bool past_end = false)
{
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int v = lidx + STRIDE * k;
        raw[k] = ldv<NTL>(&xrow[past_end ? 0 : (EXACT || v < nvec) ? v : nvec - 1]);
    }
}

// The forward's loads in a register-resident kernel whose row groups span
// STRIDE lanes (see ldv).
template <int OP, int STRIDE>
constexpr bool nt_fwd_loads()
{
    return OP == EPI_NONE && STRIDE >= 8;
}

// -inf over the window elements outside the row (unaligned rows only): only
// the window's first vector, its last and copies of the last hold any.
template <int DT, int K, int STRIDE>
__device__ __forceinline__ void mask_window(Vec (&raw)[K], int lidx, int nvec, int kfull, int head,
                                            int64_t V)
{
    constexpr int E = Traits<DT>::E;
    if (lidx == 0 && head > 0)
        mask_outside<DT>(raw[0], head, E);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (k + 1 >= kfull) {
            const int v = lidx + STRIDE * k;
            if (v >= nvec - 1)
                mask_outside<DT>(raw[k], 0, (int)(head + V - (int64_t)(nvec - 1) * E));
        }
    }
}

template <int STRIDE, bool EXACT>
__device__ __forceinline__ bool vec_valid(int k, int kfull, int lidx, int nvec)
{
    return EXACT || k < kfull || lidx + STRIDE * k < nvec;
}

// Sum over the row leaving out the target's term, re-read from memory one
// vector at a time (lane lidx takes window vectors lidx, lidx + stride, ...):
// the rare rows whose target carries more than half of the mass (p_t > 1/2).
// Kept serial and out of line so it adds no register pressure.
template <int DT>
__device__ __attribute__((noinline)) float sum_without_target(const Params &p, const Vec *xrow,
                                                              int lidx, int stride, int nvec,
                                                              int head, float mL, int vt, int jt)
{
    constexpr int E = Traits<DT>::E;
    float lx = 0.0f;
    for (int v = lidx; v < nvec; v += stride) {
        Vec r = xrow[v];
        if (!p.aligned) {
            if (v == 0 && head > 0)
                mask_outside<DT>(r, head, E);
            if (v == nvec - 1)
                mask_outside<DT>(r, 0, (int)(head + p.V - (int64_t)v * E));
        }
        lx += (v == vt) ? vec_sumexp_skip<DT>(r, mL, jt) : vec_sumexp<DT>(r, mL);
    }
    return lx;
}

// Element jt of a packed vector replaced by val (rounded to the storage type).
template <int DT>
__device__ __forceinline__ void set_elem(Vec &g, int jt, float val)
{
    constexpr int E = Traits<DT>::E;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (j == jt)
                g.w[j] = __float_as_uint(val);
    } else {
        const uint32_t b = pack2<DT>(val, val) & 0xffffu;
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (j == jt)
                g.w[j >> 1] = (j & 1) ? ((g.w[j >> 1] & 0x0000ffffu) | (b << 16))
                                      : ((g.w[j >> 1] & 0xffff0000u) | b);
    }
}

// Window geometry of one row.
struct Window {
    Vec *xrow;       // the row's first window vector
    Vec *yrow;       // the same window in the epilogue output
    int head;
    int nvec;
};

template <int DT>
__device__ __forceinline__ Window row_window(const Params &p, int64_t row)
{
    constexpr int E = Traits<DT>::E;
    const int64_t e0 = row * p.V + p.head0;
    Window w;
    w.xrow = p.x + (e0 / E);
    w.yrow = p.y + (e0 / E);
    w.head = (int)(e0 % E);
    w.nvec = (int)((w.head + p.V + E - 1) / E);
    return w;
}

// The same sum over a row held in registers (lane lidx holds window vectors
// lidx + STRIDE*k): the epilogues still hold the row when the sum is needed.
// Window elements outside the row are masked again (the backward from a given
// lse has not masked them).  Only the rare dominant-target rows take it.
template <int DT, int K, int STRIDE, bool EXACT>
__device__ __forceinline__ float regs_sum_without_target(const Params &p, const Vec (&raw)[K],
                                                         const Window &w, int lidx, int kfull,
                                                         float mL, int vt, int jt)
{
    constexpr int E = Traits<DT>::E;
    const bool masked = !EXACT && !p.aligned;
    float lx = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int v = lidx + STRIDE * k;
        Vec x = raw[k];
        if (masked) {
            if (k == 0 && lidx == 0 && w.head > 0)
                mask_outside<DT>(x, w.head, E);
            if (k + 1 >= kfull && v >= w.nvec - 1)
                mask_outside<DT>(x, 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
        }
        float e = vec_sumexp<DT>(x, mL);
        if (v == vt)
            e = vec_sumexp_skip<DT>(x, mL, jt);
        lx += vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec) ? e : 0.0f;
    }
    return lx;
}

// The gradient scale of a row: 1/M (mean) or 1, times the upstream gradient
// (per row for none, one value otherwise) when one is given.
__device__ __forceinline__ float row_scale(const Params &p, int64_t row)
{
    if (!p.dloss)
        return p.c;
    return p.c * p.dloss[p.dloss_per_row ? row : 0];
}

// Row state carried by the register pipeline: the row in raw[] was loaded
// (by the previous iteration) from window w.
struct RowRef {
    int64_t row;     // the row held (clamped to a real row for idle lanes)
    bool active;     // this lane's row is a real row
    bool past_end;   // no row follows (wave-uniform): its loads read one vector
    int64_t t;       // its target, -1 for idle lanes
    float c;         // gradient scale of the row (gradient epilogues)
    float lse;       // given log-sum-exp (EPI_LSE_GRAD)
    Window w;
};

// The "next row" after a wavefront's or workgroup's last: the last row again,
// marked so that the pipeline's loads of it (kept unconditional) all read the
// window's first vector -- one cache line per load instead of the whole row
// fetched again (a row per wavefront at the end of every launch: 16 MB for
// the 32768 x 4096 fp32 forward, 64 MB for the LM head's fused backward).
__device__ __forceinline__ RowRef past_end(const RowRef &last)
{
    RowRef r = last;
    r.past_end = true;
    return r;
}

// Window vector v of `next` for lane loads (clamped to the window; the first
// vector past the end).
template <bool EXACT>
__device__ __forceinline__ int next_vec(const RowRef &next, int v)
{
    return next.past_end ? 0 : (EXACT || v < next.w.nvec) ? v : next.w.nvec - 1;
}

// One pipeline step on a row held in registers (K vectors per lane, lane lidx
// of STRIDE lanes): the loads of `next` are issued as soon as the registers
// are free (during the sum pass for the forward; right after each gradient
// vector is stored for the fused backward), so memory stays busy while this
// row is reduced and written.  After the last row, `next` is that row
// marked past_end: its loads (kept unconditional) all read the window's first
// vector, and their values are never used.
// Returns the row's loss (same in every lane).
template <int DT, int K, int STRIDE, int OP, bool EXACT, class Red>
__device__ __forceinline__ float pipeline_step(const Params &p, Red &red, Vec (&raw)[K],
                                               const RowRef &cur, const RowRef &next, int lidx,
                                               int kfull)
{
    constexpr int E = Traits<DT>::E;
    constexpr bool BWD = OP != EPI_NONE;
    const Window &w = cur.w;
    const TargetPos tp = target_pos<DT>(cur.t, p.V, w.head);
    const bool masked = !EXACT && !p.aligned;
    // The target's logit.  Lane vt mod STRIDE of the row holds it in vector
    // k = vt / STRIDE.  In the epilogues of rows that span a whole wavefront
    // or workgroup (STRIDE >= 64) that k is the same for every lane: once the
    // fold is done, the owner takes the logit from its registers (which
    // still hold the row) and shares it (readlane, or the LDS slot of the
    // cross-wave combine).  A load from memory there made every lane wait for
    // all the row's loads before its fold could start: the value is uniform,
    // and moving it to a scalar register waited for the load, which completes
    // after every load issued before it.  The forward (its registers already
    // hold the next row), the backward from a given lse (it has no fold: its
    // epilogue starts as the row's vectors arrive, and taking the logit from
    // the registers first made it wait for the whole row, 17 % slower on the
    // classifier rows) and narrower rows read it from memory.
    //
    // Forwards of short rows read with non-temporal loads (XT_FOLD) instead
    // pick the target's vector as it is folded: a line loaded
    // non-temporally may be gone from the cache by the time the logit's own
    // load arrives, which then fetches it from memory a second time.
    // Measured per launch (~540 MB): fp32 rows of 512 bytes over 8 lanes
    // 91.4 -> 87.0 us, bf16 rows of 512 bytes over 8 lanes 96.2 -> 92.4,
    // fp32 rows of 32-128 vectors over 16-32 lanes 1.6-3 % faster; slower
    // for 16-bit rows over 16 lanes x 2 vectors (6 %) and misaligned f16
    // rows of 125 vectors over 32 lanes (5 %), which keep the load.
    constexpr bool XT_REGS = BWD && OP != EPI_LSE_GRAD && STRIDE >= 64;
    constexpr bool XT_FOLD =
        nt_fwd_loads<OP, STRIDE>() && (DT == DT_F32 ? STRIDE <= 32 : STRIDE == 8);
    constexpr bool FOLD2 = !BWD;
    // The epilogues of exact workgroup tiles refill with non-temporal loads
    // (per launch: LM head fused backward 1.640 -> 1.613 ms, its softmax
    // 1.616 -> 1.597, fp32 16384 x 32768 fused backward 811 -> 791 us), and
    // so does the softmax of exact register rows, whose output goes to
    // another buffer (32768 x 4096 fp32: 200 -> 190 us).  The fused backward
    // of register rows of one wavefront measured 6 % slower with them (32768
    // x 4096 fp32), misaligned rows 2-7 % (the stress rows' fused backward
    // and softmax, fp32 2001 and f16 999 wide softmax), the backward from a
    // given lse no faster.
    constexpr bool NT_EPI =
        BWD && EXACT && (STRIDE > 64 || OP == EPI_SOFTMAX || OP == EPI_LOGSOFTMAX);
    const int kt_own = tp.valid ? tp.vt / STRIDE : -1;
    const bool xt_owner = tp.valid && lidx == tp.vt % STRIDE;
    const int owner_lane = tp.valid ? tp.vt % STRIDE : 0;
    float xt_own = 0.0f;
    float xt = __builtin_nanf("");
    if constexpr (!XT_REGS && !XT_FOLD)
        xt = tp.valid ? load_logit<DT>(p, cur.row, cur.t) : __builtin_nanf("");
    auto take_xt = [&]() {
        if constexpr (XT_REGS) {
            // straight-line selects (kt_own is uniform): branches here made
            // the compiler spill the row's registers
            Vec tv = raw[0];
#pragma unroll
            for (int k = 1; k < K; ++k) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tv.w[i] = k == kt_own ? raw[k].w[i] : tv.w[i];
            }
            xt_own = vec_elem_dyn<DT>(tv, tp.jt);
        }
    };
    // after the combine (which, across wavefronts, also carried the logit)
    auto shared_xt = [&]() {
        if constexpr (XT_REGS) {
            float sh;
            if constexpr (STRIDE > 64)
                sh = red.xt();
            else
                sh = red.share_xt(xt_own, owner_lane);
            xt = tp.valid ? sh : __builtin_nanf("");
        }
    };

    float m, s;
    if constexpr (OP == EPI_LSE_GRAD) {
        // the row's statistics are given: exp(x - lse) = 2^((x - m) log2 e - log2 s)
        // with m = lse and s = 1
        m = cur.lse;
        s = 1.0f;
    } else if constexpr (FOLD2) {
        // Forwards: the lane's max over its vectors first, then the sum
        // against it, each register refilled with the next row's vector once
        // it is summed -- no rescale of the running sum per vector (per
        // launch: fp32 rows 2-4.5 % faster, e.g. 2M x 64 104 -> 100 us; 16-bit
        // rows 2-10 %, e.g. bf16 128K x 2000 98 -> 89 us, f16 256K x 1000 106
        // -> 97 us, although the second pass widens the elements again).
        float ml = -__builtin_inff();
        const int kt_sel = xt_owner ? kt_own : -1;   // XT_FOLD: the owner's target vector
        Vec tv = {};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = lidx + STRIDE * k;
            if (masked) {
                if (k == 0 && lidx == 0 && w.head > 0)
                    mask_outside<DT>(raw[k], w.head, E);
                if (k + 1 >= kfull && v >= w.nvec - 1)
                    mask_outside<DT>(raw[k], 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
            }
            if constexpr (XT_FOLD) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tv.w[i] = k == kt_sel ? raw[k].w[i] : tv.w[i];
            }
            const bool valid = vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec);
            ml = valid ? vec_max<DT>(raw[k], ml) : ml;
        }
        const float mlL = ml == -__builtin_inff() ? 0.0f : ml * kLog2e;
        float sl = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = lidx + STRIDE * k;
            const float e = vec_sumexp<DT>(raw[k], mlL);
            sl += vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec) ? e : 0.0f;
            raw[k] = ldv<nt_fwd_loads<OP, STRIDE>()>(&next.w.xrow[next_vec<EXACT>(next, v)]);
            // keep each load after the use of the register it refills
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (STRIDE > 64)
            red.combine(ml, sl, m, s, xt_own, xt_owner);
        else
            red.combine(ml, sl, m, s);
        if constexpr (XT_FOLD) {
            const float own = vec_elem_dyn<DT>(tv, tp.jt);
            float sh;
            if constexpr (STRIDE == 64)
                sh = red.share_xt(own, owner_lane);
            else
                sh = group_bcast<STRIDE>(own, owner_lane);
            xt = tp.valid ? sh : __builtin_nanf("");
        }
    } else if constexpr (BWD && DT == DT_F16) {
        // The epilogues issue the next row's loads only as they store, so the
        // fold may take two passes over the registers: the lane's max (two
        // fp16 elements per instruction), then its sum against that max, with
        // no per-vector rescale.  Measured: 2 % faster than the one-pass fold
        // for the fp16 stress rows; for bf16 (no packed max) it spilled and
        // was 1 % slower, so bf16 and fp32 keep the one-pass fold.
        float ml = -__builtin_inff();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = lidx + STRIDE * k;
            if (masked) {
                if (k == 0 && lidx == 0 && w.head > 0)
                    mask_outside<DT>(raw[k], w.head, E);
                if (k + 1 >= kfull && v >= w.nvec - 1)
                    mask_outside<DT>(raw[k], 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
            }
            const bool valid = vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec);
            ml = valid ? vec_max_f16_packed(raw[k], ml) : ml;
        }
        const float mlL = ml == -__builtin_inff() ? 0.0f : ml * kLog2e;
        opt_barrier<DT, K>(raw);   // widen again rather than keep widened copies
        float sl = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float e = vec_sumexp<DT>(raw[k], mlL);
            sl += vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec) ? e : 0.0f;
        }
        take_xt();
        if constexpr (STRIDE > 64)
            red.combine(ml, sl, m, s, xt_own, xt_owner);
        else
            red.combine(ml, sl, m, s);
        shared_xt();
    } else {
        // One pass: each vector is folded into the lane's running (max, sum)
        // as it arrives -- the sum is rescaled by 2^((m_old - m_new) log2 e)
        // when the max grows -- and (forward) its registers are refilled at
        // once with the next row's vector.
        float m_run = -__builtin_inff();
        float s_run = 0.0f;
        const int kt_sel = xt_owner ? kt_own : -1;   // XT_FOLD: the owner's target vector
        Vec tv = {};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = lidx + STRIDE * k;
            Vec x = raw[k];
            if (masked) {
                if (k == 0 && lidx == 0 && w.head > 0)
                    mask_outside<DT>(x, w.head, E);
                if (k + 1 >= kfull && v >= w.nvec - 1)
                    mask_outside<DT>(x, 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
            }
            if constexpr (BWD) {
                if (masked)
                    raw[k] = x;
            }
            if constexpr (XT_FOLD) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tv.w[i] = k == kt_sel ? x.w[i] : tv.w[i];
            }
            const bool valid = vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec);
            const float mn = vec_max<DT>(x, m_run);
            const float mnL = mn == -__builtin_inff() ? 0.0f : mn * kLog2e;
            const float add = vec_sumexp<DT>(x, mnL);
            const float s_new = __builtin_fmaf(rescale_to(s_run, m_run, mn), 1.0f, add);
            s_run = valid ? s_new : s_run;
            m_run = valid ? mn : m_run;
            if constexpr (!BWD) {
                raw[k] = ldv<nt_fwd_loads<OP, STRIDE>()>(&next.w.xrow[next_vec<EXACT>(next, v)]);
                // keep each load after the use of the register it refills
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        take_xt();
        if constexpr (STRIDE > 64)
            red.combine(m_run, s_run, m, s, xt_own, xt_owner);
        else
            red.combine(m_run, s_run, m, s);
        shared_xt();
        if constexpr (XT_FOLD) {
            const float own = vec_elem_dyn<DT>(tv, tp.jt);
            float sh;
            if constexpr (STRIDE == 64)
                sh = red.share_xt(own, owner_lane);
            else
                sh = group_bcast<STRIDE>(own, owner_lane);
            xt = tp.valid ? sh : __builtin_nanf("");
        }
    }
    const float mL = m * kLog2e;

    const float et = fast_exp2(__builtin_fmaf(xt, kLog2e, -mL));
    const bool accurate = tp.valid && et > 0.5f * s;
    float s_excl = s - et;
    if (accurate) {
        // the epilogues still hold the row in registers; the forward has
        // refilled them with the next row and reads this one again
        if constexpr (BWD) {
            opt_barrier<DT, K>(raw);   // widen again rather than keep the fold's copies
            s_excl = red.sum_excl(regs_sum_without_target<DT, K, STRIDE, EXACT>(
                p, raw, w, lidx, kfull, mL, tp.vt, tp.jt));
        } else {
            s_excl = red.sum_excl(sum_without_target<DT>(p, w.xrow, lidx, STRIDE, w.nvec, w.head,
                                                         mL, tp.vt, tp.jt));
        }
    }
    const float c = cur.c;
    const RowResult rr = row_result(tp.valid, m, xt, et, s, s_excl, accurate, c);
    const float log2s = OP == EPI_LSE_GRAD ? 0.0f : __log2f(s);
    if (OP != EPI_LSE_GRAD && p.lse_out && cur.active && lidx == 0)
        p.lse_out[cur.row] = m + kLn2 * log2s;

    if constexpr (BWD) {
        opt_barrier<DT, K>(raw);
        constexpr int EOP = OP == EPI_LSE_GRAD ? EPI_GRAD : OP;
        const EpiCoef<DT> ec = epi_coef<DT, EOP>(m, mL, log2s, c);
        const int kt = (EOP == EPI_GRAD && tp.valid) ? tp.vt / STRIDE : -1;
        const bool is_owner = tp.valid && lidx == tp.vt % STRIDE;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = lidx + STRIDE * k;
            Vec g = epi_vec<DT, EOP>(raw[k], ec);
            if (k == kt) {
                if (is_owner)
                    set_elem<DT>(g, tp.jt, rr.gt);
            }
            if (cur.active && vec_valid<STRIDE, EXACT>(k, kfull, lidx, w.nvec))
                store_grad<DT>(w.yrow, v, g, w.head, p.V, EXACT || p.aligned);
            raw[k] = ldv<NT_EPI>(&next.w.xrow[next_vec<EXACT>(next, v)]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    red.next_row();
    return rr.loss;
}

// --------------------------------------------- end of kernel: mean / sum
// Every workgroup stores its fp64 loss sum (its wavefronts' sums added in
// wavefront order) in its own slot, and the slots
// are added in index order by one wavefront: the last workgroup of the same
// launch (finish_in_kernel, below), or, where the launch has no counter (a
// graph capture, split rows), a second one-wavefront kernel on the same
// stream.  The order of every addition is fixed by the launch shape, so the
// two forms give the same bits.

// Sum over the 64 lanes in a fixed butterfly order; every lane gets the sum.
__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Adds nunits partial sums in a fixed order with one wavefront (all lanes
// get the total).
__device__ __forceinline__ double sum_partials(const double *partials, unsigned nunits, int lane)
{
    double acc = 0.0;
    for (unsigned base = 0; base < nunits; base += 64 * 8) {
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned i = base + (unsigned)lane + 64u * j;
            v[j] = i < nunits ? partials[i] : 0.0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc += v[j];
    }
    return wave_sum_f64(acc);
}

// The final sum of a mean or sum in the launch that made the partials:
// each workgroup, once all its wavefronts have published theirs, takes a
// ticket (an integer counter); the one that takes the last adds all nunits
// partials in the same fixed order as the second-kernel form, so the result
// is that form's bit for bit, and puts the counter back to zero for the
// next launch.  No fences: each partial is stored through to memory (a
// system-scope store that no cache keeps) and waited for before the
// workgroup's ticket, and the last workgroup reads the partials the same
// way (system-scope loads that miss every cache); an agent-scope release
// would write back the whole L2 instead.
__device__ __forceinline__ void publish_partial(const Params &p, unsigned idx, double v)
{
    if (p.ticket)
        __hip_atomic_store(&p.partials[idx], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else
        p.partials[idx] = v;
}

__device__ __forceinline__ void finish_in_kernel(const Params &p, unsigned nunits, int lane,
                                                 int wave)
{
    __shared__ unsigned s_last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's partial is in memory
    __syncthreads();                                    // ... and every wavefront's
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev + 1 == gridDim.x ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last || wave != 0)
        return;
    // sum_partials' order, with loads from memory
    double acc = 0.0;
    for (unsigned base = 0; base < nunits; base += 64 * 8) {
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned i = base + (unsigned)lane + 64u * j;
            v[j] = i < nunits ? __hip_atomic_load(&p.partials[i], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_SYSTEM)
                              : 0.0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc += v[j];
    }
    const double total = wave_sum_f64(acc);
    if (lane == 0) {
        p.out[0] = (float)(total * p.out_scale);
        __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ================================================================ kernels


template <int DT, int OP>
__device__ __forceinline__ RowRef row_ref(const Params &p, int64_t row)
{
    RowRef r;
    r.active = row < p.M;
    r.past_end = false;
    r.row = r.active ? row : 0;   // idle lanes redo row 0, store nothing, drop the loss
    // The per-row scalars are read here, a step before they are used and
    // before the row's own loads: vector loads retire in order, so a late
    // load would make the wave wait for every prefetch issued before it.
    r.t = (r.active && p.targets) ? row_scalar(p.targets, r.row) : -1;
    r.c = (OP == EPI_GRAD || OP == EPI_LSE_GRAD) ? row_scale(p, r.row) : 0.0f;
    r.lse = OP == EPI_LSE_GRAD ? p.lse_in[r.row] : 0.0f;
    r.w = row_window<DT>(p, r.row);
    return r;
}

// ---- G lanes per row, row in registers ------------------------------------
// NBUF row buffers per lane: with 2, the rows a wave handles alternate between
// two register sets, so each row's loads are issued a whole row ahead.
template <int DT, int G, int K, int OP, bool EXACT, int NBUF, int NW = 4>
__global__ void __launch_bounds__(NW * 64) rows_kernel(Params p)
{
    static_assert(NBUF == 1 || NBUF == 2, "NBUF");
    constexpr int E = Traits<DT>::E;
    constexpr int GPW = 64 / G;               // rows per wavefront
    const int lane = threadIdx.x & 63;
    const int lig = lane & (G - 1);
    // wave-uniform, and known to be: keeps the row loop a scalar loop
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int kfull = (int)((p.V + E - 1) / E) / G;
    double acc = 0.0;

    // Rows of this wave: rb, rb + row_step, ... below row_end.  Interleaved:
    // the whole grid strides over the rows.  Blocked: each workgroup owns a
    // contiguous band of rows and walks it front to back.
    int64_t rb, row_step, row_end;
    if (p.blocked) {
        const int64_t per_wg = (int64_t)nwaves * GPW;
        const int64_t band = (p.M + (int64_t)gridDim.x * per_wg - 1) / ((int64_t)gridDim.x * per_wg) * per_wg;
        rb = (int64_t)blockIdx.x * band + (int64_t)wave * GPW;
        row_step = per_wg;
        row_end = (int64_t)(blockIdx.x + 1) * band < p.M ? (int64_t)(blockIdx.x + 1) * band : p.M;
    } else {
        rb = ((int64_t)blockIdx.x * nwaves + wave) * GPW;
        row_step = (int64_t)gridDim.x * nwaves * GPW;
        row_end = p.M;
    }
    auto record = [&](const RowRef &r, float loss) {
        if (r.active && lig == 0) {
            if (p.reduction == RED_NONE) {
                if (p.out)
                    p.out[r.row] = loss;
            } else {
                acc += (double)loss;
            }
        }
    };
    // the group's row in the wave's row block `base`, or fallback past the end
    auto ref_at = [&](int64_t base, const RowRef &fallback) {
        return base < row_end ? row_ref<DT, OP>(p, base + lane / G) : past_end(fallback);
    };
    GroupRed<G> red;
    if (rb < row_end) {
        RowRef a = row_ref<DT, OP>(p, rb + lane / G);
        Vec ra[K];
        issue_loads<DT, K, G, EXACT, nt_fwd_loads<OP, G>()>(ra, a.w.xrow, lig, a.w.nvec);
        if constexpr (NBUF == 1) {
            for (; rb < row_end; rb += row_step) {
                const RowRef an = ref_at(rb + row_step, a);
                record(a, pipeline_step<DT, K, G, OP, EXACT>(p, red, ra, a, an, lig, kfull));
                a = an;
            }
        } else {
            RowRef b = ref_at(rb + row_step, a);
            Vec rbuf[K];
            issue_loads<DT, K, G, EXACT, nt_fwd_loads<OP, G>()>(rbuf, b.w.xrow, lig, b.w.nvec,
                                                                b.past_end);
            for (; rb < row_end; rb += 2 * row_step) {
                const RowRef an = ref_at(rb + 2 * row_step, a);
                record(a, pipeline_step<DT, K, G, OP, EXACT>(p, red, ra, a, an, lig, kfull));
                if (rb + row_step >= row_end)
                    break;
                const RowRef bn = ref_at(rb + 3 * row_step, b);
                record(b, pipeline_step<DT, K, G, OP, EXACT>(p, red, rbuf, b, bn, lig, kfull));
                a = an;
                b = bn;
            }
        }
    }

    if (p.reduction == RED_NONE)
        return;
    // lanes other than each group's first hold 0; the wavefronts' sums are
    // added in wavefront order into one partial per workgroup (a quarter of
    // the partials for the last workgroup to read: measured 0.2-0.7 us off
    // the 32768 x 4096 fp32 forward)
    const double wave_total = wave_sum_f64(acc);
    __shared__ double s_wave_sums[NW];
    if (lane == 0)
        s_wave_sums[wave] = wave_total;
    __syncthreads();
    if (threadIdx.x == 0) {
        double wg_total = s_wave_sums[0];
        for (int w = 1; w < nwaves; ++w)
            wg_total += s_wave_sums[w];
        publish_partial(p, blockIdx.x, wg_total);
    }
    if (p.ticket)
        finish_in_kernel(p, gridDim.x, lane, wave);
}

// ---- one row per workgroup, row in registers --------------------------------
// OCC: waves per SIMD the register allocation must leave room for (4 with 8
// waves per workgroup: two workgroups per CU, each holding its own row).
template <int DT, int W, int K, int OP, bool EXACT, int OCC = 1>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
wg_kernel(Params p)
{
    constexpr int E = Traits<DT>::E;
    constexpr int NT = W * 64;
    __shared__ float s_max[2][W], s_sum[2][W], s_exc[2][W], s_xt[2];
    WgRed<W> red;
    red.smax = s_max;
    red.ssum = s_sum;
    red.sexc = s_exc;
    red.sxt = s_xt;
    red.wave = threadIdx.x >> 6;
    red.lane = threadIdx.x & 63;
    red.bank = 0;
    const int kfull = (int)((p.V + E - 1) / E) / NT;
    double acc = 0.0;

    // interleaved (grid stride) or blocked (a contiguous band per workgroup)
    int64_t row, row_step, row_end;
    if (p.blocked) {
        const int64_t band = (p.M + gridDim.x - 1) / gridDim.x;
        row = (int64_t)blockIdx.x * band;
        row_step = 1;
        row_end = row + band < p.M ? row + band : p.M;
    } else {
        row = blockIdx.x;
        row_step = gridDim.x;
        row_end = p.M;
    }
    if (row < row_end) {
        RowRef cur = row_ref<DT, OP>(p, row);
        Vec raw[K];
        issue_loads<DT, K, NT, EXACT, nt_fwd_loads<OP, NT>()>(raw, cur.w.xrow, threadIdx.x,
                                                              cur.w.nvec);
        for (; row < row_end; row += row_step) {
            const bool has_next = row + row_step < row_end;
            const RowRef next = has_next ? row_ref<DT, OP>(p, row + row_step) : past_end(cur);
            const float loss =
                pipeline_step<DT, K, NT, OP, EXACT>(p, red, raw, cur, next, threadIdx.x, kfull);
            if (threadIdx.x == 0) {
                if (p.reduction == RED_NONE) {
                    if (p.out)
                        p.out[row] = loss;
                } else {
                    acc += (double)loss;
                }
            }
            cur = next;
        }
    }
    // thread 0 holds the workgroup's sum
    if (p.reduction != RED_NONE && threadIdx.x == 0)
        publish_partial(p, blockIdx.x, acc);
    if (p.ticket)
        finish_in_kernel(p, gridDim.x, threadIdx.x & 63, threadIdx.x >> 6);
}

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// ---- one row per wavefront, streamed in chunks ------------------------------
// Every wavefront walks its own rows (grid stride over wavefronts); a row is
// read in chunks of 64*K vectors folded into per-lane online (max, sum)
// pairs, then combined with DPP.  No LDS and no barriers: many wavefronts per
// CU keep memory busy.  Forward only.
template <int DT, int K>
__global__ void __launch_bounds__(256) wstream_kernel(Params p)
{
    constexpr int E = Traits<DT>::E;
    constexpr int CH = 64 * K;
    // 16-bit rows: in a row's last, partly empty chunk, vector slots wholly
    // past the row (the row is the wavefront's, so the test is uniform) are
    // neither loaded nor folded -- the folds are VALU-bound (bf16 2100 wide,
    // one half-empty chunk of 512 vectors: 166 -> 126 us per launch for 128K
    // rows); full chunks keep the branch-free code.  fp32 rows keep every load
    // in one batch: skipping made them 2-8 % slower.
    constexpr bool SKIP = DT != DT_F32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int64_t step = (int64_t)gridDim.x * nwaves;
    GroupRed<64> red;
    double acc = 0.0;

    for (int64_t row = (int64_t)blockIdx.x * nwaves + wave; row < p.M; row += step) {
        const Window w = row_window<DT>(p, row);
        const int64_t t = p.targets ? row_scalar(p.targets, row) : -1;
        const TargetPos tp = target_pos<DT>(t, p.V, w.head);
        const float xt = tp.valid ? load_logit<DT>(p, row, t) : __builtin_nanf("");
        float m_run = -__builtin_inff();
        float s_run = 0.0f;
        // one chunk of a 16-bit row; PART: the row's last, partly empty one
        // (fp32 rows: the loop below, unchanged)
        auto chunk = [&](auto part, int cb) {
            constexpr bool PART = decltype(part)::value;
            const int n = w.nvec - cb;          // window vectors from this chunk on
            const Vec *xc = w.xrow + cb;
            Vec raw[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int v = lane + 64 * k;
                if (!PART || 64 * k < n)
                    raw[k] = ldv<true>(&xc[v < n ? v : n - 1]);
                else
                    raw[k] = Vec{};
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (PART && 64 * k >= n)
                    break;
                const int v = lane + 64 * k;
                Vec x = raw[k];
                if (!p.aligned) {
                    if (cb == 0 && v == 0 && w.head > 0)
                        mask_outside<DT>(x, w.head, E);
                    if (v >= n - 1)
                        mask_outside<DT>(x, 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
                }
                const bool valid = v < n;
                const float mn = vec_max<DT>(x, m_run);
                const float mnL = mn == -__builtin_inff() ? 0.0f : mn * kLog2e;
                const float add = vec_sumexp<DT>(x, mnL);
                const float s_new = rescale_to(s_run, m_run, mn) + add;
                s_run = valid ? s_new : s_run;
                m_run = valid ? mn : m_run;
            }
        };
        if constexpr (SKIP && K >= 8) {
            // rows of 257-512 vectors: one chunk, partly empty.  Written out
            // here: through the lambda it measured 7 % slower (bf16 2100
            // wide: 135 against 126 us), and a second, branch-free copy cost
            // registers (occupancy 7 -> 4).
            for (int cb = 0; cb < w.nvec; cb += CH) {
                const int n = w.nvec - cb;
                const Vec *xc = w.xrow + cb;
                Vec raw[K];
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int v = lane + 64 * k;
                    if (64 * k < n)
                        raw[k] = ldv<true>(&xc[v < n ? v : n - 1]);
                    else
                        raw[k] = Vec{};
                }
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (64 * k >= n)
                        break;
                    const int v = lane + 64 * k;
                    Vec x = raw[k];
                    if (!p.aligned) {
                        if (cb == 0 && v == 0 && w.head > 0)
                            mask_outside<DT>(x, w.head, E);
                        if (v >= n - 1)
                            mask_outside<DT>(x, 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
                    }
                    const bool valid = v < n;
                    const float mn = vec_max<DT>(x, m_run);
                    const float mnL = mn == -__builtin_inff() ? 0.0f : mn * kLog2e;
                    const float add = vec_sumexp<DT>(x, mnL);
                    const float s_new = rescale_to(s_run, m_run, mn) + add;
                    s_run = valid ? s_new : s_run;
                    m_run = valid ? mn : m_run;
                }
            }
        } else if constexpr (SKIP) {
            for (int cb = 0; cb < w.nvec; cb += CH) {
                if (w.nvec - cb < CH)
                    chunk(BoolTag<true>{}, cb);
                else
                    chunk(BoolTag<false>{}, cb);
            }
        } else {
            for (int cb = 0; cb < w.nvec; cb += CH) {
                const int n = w.nvec - cb;          // window vectors from this chunk on
                const Vec *xc = w.xrow + cb;
                Vec raw[K];
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int v = lane + 64 * k;
                    raw[k] = ldv<true>(&xc[v < n ? v : n - 1]);
                }
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int v = lane + 64 * k;
                    Vec x = raw[k];
                    if (!p.aligned) {
                        if (cb == 0 && v == 0 && w.head > 0)
                            mask_outside<DT>(x, w.head, E);
                        if (v >= n - 1)
                            mask_outside<DT>(x, 0, (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E));
                    }
                    const bool valid = v < n;
                    const float mn = vec_max<DT>(x, m_run);
                    const float mnL = mn == -__builtin_inff() ? 0.0f : mn * kLog2e;
                    const float add = vec_sumexp<DT>(x, mnL);
                    const float s_new = rescale_to(s_run, m_run, mn) + add;
                    s_run = valid ? s_new : s_run;
                    m_run = valid ? mn : m_run;
                }
            }
        }
        float m, s;
        red.combine(m_run, s_run, m, s);
        const float mL = m * kLog2e;
        const float et = fast_exp2(__builtin_fmaf(xt, kLog2e, -mL));
        const bool accurate = tp.valid && et > 0.5f * s;
        float s_excl = s - et;
        if (accurate)
            s_excl = red.sum_excl(sum_without_target<DT>(p, w.xrow, lane, 64, w.nvec, w.head, mL,
                                                         tp.vt, tp.jt));
        const RowResult rr = row_result(tp.valid, m, xt, et, s, s_excl, accurate, p.c);
        if (lane == 0) {
            if (p.lse_out)
                p.lse_out[row] = m + kLn2 * __log2f(s);
            if (p.reduction == RED_NONE) {
                if (p.out)
                    p.out[row] = rr.loss;
            } else {
                acc += (double)rr.loss;
            }
        }
    }
    if (p.reduction == RED_NONE)
        return;
    // lane 0 holds the wavefront's sum; the workgroup's are added in
    // wavefront order into one partial per workgroup (as the rows kernels do)
    __shared__ double s_wave_sums[4];   // 256 threads
    if (lane == 0)
        s_wave_sums[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double wg_total = s_wave_sums[0];
        for (int w = 1; w < nwaves; ++w)
            wg_total += s_wave_sums[w];
        publish_partial(p, blockIdx.x, wg_total);
    }
    if (p.ticket)
        finish_in_kernel(p, gridDim.x, lane, wave);
}

// ---- one row per workgroup, streamed in chunks ---------------------------------
template <int DT, int W, int K, int OP>
__global__ void __launch_bounds__(W * 64) stream_kernel(Params p)
{
    constexpr bool BWD = OP != EPI_NONE;
    constexpr int E = Traits<DT>::E;
    constexpr int NT = W * 64;
    constexpr int CH = NT * K;                  // vectors per chunk
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    __shared__ float s_max[W], s_sum[W], s_exc[W], s_xt;
    double acc = 0.0;

    for (int64_t row = blockIdx.x; row < p.M; row += gridDim.x) {
        const Window w = row_window<DT>(p, row);
        const int64_t t = p.targets ? row_scalar(p.targets, row) : -1;
        const TargetPos tp = target_pos<DT>(t, p.V, w.head);

        float m, s, xt;
        // the sum of the terms other than the target's, when pass 1 gives it
        // (p_t > 1/2 then needs no second read of the row)
        bool have_excl = false;
        float s_other = 0.0f;
        if constexpr (OP == EPI_LSE_GRAD) {
            // statistics given: m = lse, s = 1
            m = p.lse_in[row];
            s = 1.0f;
            xt = tp.valid ? load_logit<DT>(p, row, t) : __builtin_nanf("");
        } else {
            // pass 1: online (max, sum) per lane, rescaled once per chunk; the
            // max takes every element, the sum every element but the target
            float m_run = -__builtin_inff();
            float s_run = 0.0f;
            // 16-bit forwards: in a row's last, partly empty chunk, the vector
            // slots wholly past the row for a wavefront (a uniform test) are
            // neither loaded nor folded -- the folds are VALU-bound; full
            // chunks, fp32 rows and the epilogues take the loop below as it
            // was
            constexpr bool SKIP = DT != DT_F32 && OP == EPI_NONE;
            const int wfirst = __builtin_amdgcn_readfirstlane(64 * wave);
            auto chunk = [&](auto part, int cb) {
                constexpr bool PART = decltype(part)::value;
                Vec raw[K];
                const int n = w.nvec - cb;
                const int kfull = n >= CH ? K : n / NT;
                load_window<DT, K, NT, !BWD, PART>(raw, w.xrow + cb, tid, n, kfull,
                                                   cb == 0 ? w.head : 0,
                                                   cb == 0 ? p.V : p.V + w.head - (int64_t)cb * E,
                                                   p.aligned != 0, wfirst);
                float tval = -__builtin_inff();
                if (tp.valid && tp.vt >= cb && tp.vt < cb + CH) {
                    const int off = tp.vt - cb;
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        if (off == tid + NT * k) {
                            tval = vec_elem_dyn<DT>(raw[k], tp.jt);
                            s_xt = tval;
                            set_elem<DT>(raw[k], tp.jt, -__builtin_inff());
                        }
                }
                float cm = fmaxf(m_run, tval);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (PART && wfirst + NT * k >= n)
                        break;
                    cm = vec_max<DT>(raw[k], cm);
                }
                if (cm != -__builtin_inff()) {
                    const float cmL = cm * kLog2e;
                    float add = 0.0f;
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        if (PART && wfirst + NT * k >= n)
                            break;
                        const float e = vec_sumexp<DT>(raw[k], cmL);
                        add += vec_valid<NT>(k, kfull, tid, n) ? e : 0.0f;
                    }
                    s_run = s_run * fast_exp2((m_run - cm) * kLog2e) + add;
                    m_run = cm;
                }
            };
            if constexpr (SKIP) {
                for (int cb = 0; cb < w.nvec; cb += CH) {
                    if (w.nvec - cb < CH)
                        chunk(BoolTag<true>{}, cb);
                    else
                        chunk(BoolTag<false>{}, cb);
                }
            } else {
                for (int cb = 0; cb < w.nvec; cb += CH) {
                    Vec raw[K];
                    const int kfull = (w.nvec - cb) >= CH ? K : (w.nvec - cb) / NT;
                    // the chunk is a window of its own: the row's head lies in chunk 0,
                    // and its end is at element head + V - cb*E of the chunk
                    load_window<DT, K, NT, !BWD>(raw, w.xrow + cb, tid, w.nvec - cb, kfull,
                                                 cb == 0 ? w.head : 0,
                                                 cb == 0 ? p.V : p.V + w.head - (int64_t)cb * E,
                                                 p.aligned != 0);
                    // the lane holding the target keeps its logit aside and drops it
                    // from the vector: it enters the max below, not the sum
                    float tval = -__builtin_inff();
                    if (tp.valid && tp.vt >= cb && tp.vt < cb + CH) {
                        const int off = tp.vt - cb;
#pragma unroll
                        for (int k = 0; k < K; ++k)
                            if (off == tid + NT * k) {
                                tval = vec_elem_dyn<DT>(raw[k], tp.jt);
                                s_xt = tval;
                                set_elem<DT>(raw[k], tp.jt, -__builtin_inff());
                            }
                    }
                    float cm = fmaxf(m_run, tval);
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        cm = vec_max<DT>(raw[k], cm);
                    if (cm != -__builtin_inff()) {
                        const float cmL = cm * kLog2e;
                        float add = 0.0f;
#pragma unroll
                        for (int k = 0; k < K; ++k) {
                            const float e = vec_sumexp<DT>(raw[k], cmL);
                            add += vec_valid<NT>(k, kfull, tid, w.nvec - cb) ? e : 0.0f;
                        }
                        // the old sum is scaled by 2^(m_old - m_new); m_old = -inf gives 0
                        s_run = s_run * fast_exp2((m_run - cm) * kLog2e) + add;
                        m_run = cm;
                    }
                }
            }
            float wm = group_reduce<64>(m_run, OpMax());
            if (lane == 0)
                s_max[wave] = wm;
            __syncthreads();
            m = s_max[0];
#pragma unroll
            for (int i = 1; i < W; ++i)
                m = fmaxf(m, s_max[i]);
            const float mL = m * kLog2e;
            xt = tp.valid ? s_xt : __builtin_nanf("");
            // every lane's sum, moved to the row max
            float ls = (m_run == -__builtin_inff()) ? 0.0f : s_run * fast_exp2(m_run * kLog2e - mL);
            ls = group_reduce<64>(ls, OpSum());
            if (lane == 0)
                s_sum[wave] = ls;
            __syncthreads();
            s_other = s_sum[0];
#pragma unroll
            for (int i = 1; i < W; ++i)
                s_other += s_sum[i];
            have_excl = true;
            s = s_other;
        }
        const float mL = m * kLog2e;

        const float et = fast_exp2(__builtin_fmaf(xt, kLog2e, -mL));
        if (have_excl && tp.valid)
            s = s_other + et;
        const bool accurate = tp.valid && et > 0.5f * s;
        float s_excl = have_excl ? s_other : s - et;
        if (accurate && !have_excl) {
            // re-read the row and sum every term but the target's
            float lx = 0.0f;
            for (int cb = 0; cb < w.nvec; cb += CH) {
                Vec raw[K];
                const int kfull = (w.nvec - cb) >= CH ? K : (w.nvec - cb) / NT;
                load_window<DT, K, NT>(raw, w.xrow + cb, tid, w.nvec - cb, kfull,
                                       cb == 0 ? w.head : 0,
                                       cb == 0 ? p.V : p.V + w.head - (int64_t)cb * E,
                                       p.aligned != 0);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const float e = (cb + tid + NT * k == tp.vt) ? vec_sumexp_skip<DT>(raw[k], mL, tp.jt)
                                                                 : vec_sumexp<DT>(raw[k], mL);
                    lx += vec_valid<NT>(k, kfull, tid, w.nvec - cb) ? e : 0.0f;
                }
            }
            lx = group_reduce<64>(lx, OpSum());
            if (lane == 0)
                s_exc[wave] = lx;
            __syncthreads();
            s_excl = s_exc[0];
#pragma unroll
            for (int i = 1; i < W; ++i)
                s_excl += s_exc[i];
        }
        const float c = row_scale(p, row);
        const RowResult rr = row_result(tp.valid, m, xt, et, s, s_excl, accurate, c);
        const float log2s = OP == EPI_LSE_GRAD ? 0.0f : __log2f(s);
        if (OP != EPI_LSE_GRAD && p.lse_out && tid == 0)
            p.lse_out[row] = m + kLn2 * log2s;

        if constexpr (BWD) {
            // pass 2: re-read the row and write the epilogue
            constexpr int EOP = OP == EPI_LSE_GRAD ? EPI_GRAD : OP;
            const EpiCoef<DT> ec = epi_coef<DT, EOP>(m, mL, log2s, c);
            for (int cb = 0; cb < w.nvec; cb += CH) {
                Vec raw[K];
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int v = cb + tid + NT * k;
                    if (v < w.nvec)
                        raw[k] = ldv(&w.xrow[v]);
                }
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int v = cb + tid + NT * k;
                    if (v < w.nvec) {
                        Vec g = epi_vec<DT, EOP>(raw[k], ec);
                        if (EOP == EPI_GRAD && v == tp.vt)
                            set_elem<DT>(g, tp.jt, rr.gt);
                        store_grad<DT>(w.yrow, v, g, w.head, p.V, p.aligned);
                    }
                }
            }
        }
        if (tid == 0) {
            if (p.reduction == RED_NONE) {
                if (p.out)
                    p.out[row] = rr.loss;
            } else {
                acc += (double)rr.loss;
            }
        }
        __syncthreads();   // s_xt and the LDS partials are reused by the next row
    }
    if (p.reduction != RED_NONE && tid == 0)
        publish_partial(p, blockIdx.x, acc);
    if (p.ticket)
        finish_in_kernel(p, gridDim.x, tid & 63, tid >> 6);
}


// ---- split rows: several workgroups per row ---------------------------------
// For few long rows: workgroup b takes slice b % S of row b / S (slice_vecs
// window vectors).  A first kernel leaves each slice's (max, sum of
// exp(x - max)) with the target element left out; the epilogue kernel
// combines a row's S pairs in a fixed order (every workgroup of the row
// computes the same combine) and writes its slice.  Leaving the target out
// gives the sum of the other terms exactly, so the dominant-target form of
// the loss and of the target's gradient needs no second read.

template <int DT, int W, int K>
__global__ void __launch_bounds__(W * 64) split_stats_kernel(Params p)
{
    constexpr int E = Traits<DT>::E;
    constexpr int NT = W * 64;
    constexpr int CH = NT * K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    __shared__ float s_m[W], s_s[W];
    const int64_t row = blockIdx.x / p.S;
    const int slice = blockIdx.x % p.S;
    const Window w = row_window<DT>(p, row);
    const int64_t t = p.targets ? row_scalar(p.targets, row) : -1;
    const TargetPos tp = target_pos<DT>(t, p.V, w.head);
    const int v0 = slice * p.slice_vecs;
    const int v1 = v0 + p.slice_vecs < w.nvec ? v0 + p.slice_vecs : w.nvec;
    const int tail_n = (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E);
    // the slice holding the target saves its logit for the later kernels
    if (tid == 0 && tp.vt >= v0 && tp.vt < v1)
        p.rowx[row] = load_logit<DT>(p, row, t);
    float m_run = -__builtin_inff();
    float s_run = 0.0f;
    for (int cb = v0; cb < v1; cb += CH) {
        Vec raw[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = cb + tid + NT * k;
            raw[k] = ldv(&w.xrow[v < v1 ? v : v1 - 1]);
        }
        float cm = m_run;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = cb + tid + NT * k;
            if (v == 0 && w.head > 0)
                mask_outside<DT>(raw[k], w.head, E);
            if (v == w.nvec - 1)
                mask_outside<DT>(raw[k], 0, tail_n);
            if (v == tp.vt)
                set_elem<DT>(raw[k], tp.jt, -__builtin_inff());
            cm = v < v1 ? vec_max<DT>(raw[k], cm) : cm;
        }
        if (cm != -__builtin_inff()) {
            const float cmL = cm * kLog2e;
            float add = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float e = vec_sumexp<DT>(raw[k], cmL);
                add += (cb + tid + NT * k) < v1 ? e : 0.0f;
            }
            s_run = rescale_to(s_run, m_run, cm) + add;
            m_run = cm;
        }
    }
    const float wm = group_reduce<64>(m_run, OpMax());
    const float ws = group_reduce<64>(rescale_to(s_run, m_run, wm), OpSum());
    if (lane == 0) {
        s_m[wave] = wm;
        s_s[wave] = ws;
    }
    __syncthreads();
    if (tid == 0) {
        float m = s_m[0];
#pragma unroll
        for (int i = 1; i < W; ++i)
            m = fmaxf(m, s_m[i]);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < W; ++i)
            s += rescale_to(s_s[i], s_m[i], m);
        p.stats[2 * blockIdx.x] = m;
        p.stats[2 * blockIdx.x + 1] = s;
    }
}

// The row's statistics from its S slice pairs, in a fixed order, by one
// wavefront (every lane gets them): max and sum over all terms but the target.
__device__ __forceinline__ void combine_slices(const Params &p, int64_t row, int lane,
                                               float &m_ex, float &s_ex)
{
    const float *st = p.stats + 2 * row * p.S;
    const float mi = lane < p.S ? st[2 * lane] : -__builtin_inff();
    const float si = lane < p.S ? st[2 * lane + 1] : 0.0f;
    m_ex = group_reduce<64>(mi, OpMax());
    s_ex = group_reduce<64>(rescale_to(si, mi, m_ex), OpSum());
}

// OP == EPI_NONE: one 64-thread workgroup per row (b = row) finishing the
// forward; otherwise workgroup b writes the epilogue over slice b % S of row
// b / S.  The loss, lse and partial sums are written by slice 0.
template <int DT, int W, int K, int OP>
__global__ void __launch_bounds__(W * 64) split_epi_kernel(Params p)
{
    constexpr int E = Traits<DT>::E;
    constexpr int NT = W * 64;
    constexpr int CH = NT * K;
    constexpr int EOP = OP == EPI_LSE_GRAD ? EPI_GRAD : OP;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    __shared__ float s_row[3];
    const int64_t row = OP == EPI_NONE ? (int64_t)blockIdx.x : (int64_t)(blockIdx.x / p.S);
    const int slice = OP == EPI_NONE ? 0 : (int)(blockIdx.x % p.S);
    const Window w = row_window<DT>(p, row);
    const int64_t t = p.targets ? row_scalar(p.targets, row) : -1;
    const TargetPos tp = target_pos<DT>(t, p.V, w.head);
    const float c = (EOP == EPI_GRAD) ? row_scale(p, row) : 0.0f;
    const int v0 = slice * p.slice_vecs;
    const int v1 = v0 + p.slice_vecs < w.nvec ? v0 + p.slice_vecs : w.nvec;
    const bool owner = tp.vt >= v0 && tp.vt < v1;   // this slice holds the target
    if (wave == 0) {
        // The target logit: saved by the statistics kernel; for the backward
        // from a given lse only the owner needs it (it reads it before any
        // store of its own, and saves it for the fix).  Other slices of an
        // in-place call may already have overwritten it.
        float xt = __builtin_nanf("");
        if constexpr (OP == EPI_LSE_GRAD) {
            if (owner) {
                xt = load_logit<DT>(p, row, t);
                if (lane == 0)
                    p.rowx[row] = xt;
            }
        } else if (tp.valid) {
            xt = p.rowx[row];
        }
        float m, s, s_excl;
        if constexpr (OP == EPI_LSE_GRAD) {
            m = p.lse_in[row];
            s = 1.0f;
            s_excl = 0.0f;   // unused: the target's gradient is (p_t - 1) c, refined later
        } else {
            float m_ex, s_ex;
            combine_slices(p, row, lane, m_ex, s_ex);
            m = tp.valid ? fmaxf(m_ex, xt) : m_ex;
            s_excl = rescale_to(s_ex, m_ex, m);
            s = s_excl;
        }
        const float mL = m * kLog2e;
        const float et = tp.valid ? fast_exp2(__builtin_fmaf(xt, kLog2e, -mL)) : 0.0f;
        if constexpr (OP != EPI_LSE_GRAD)
            s += et;
        else
            s_excl = s - et;
        const bool accurate = OP != EPI_LSE_GRAD && tp.valid && et > 0.5f * s;
        const RowResult rr = row_result(tp.valid, m, xt, et, s, s_excl, accurate, c);
        const float log2s = OP == EPI_LSE_GRAD ? 0.0f : __log2f(s);
        if (lane == 0) {
            s_row[0] = m;
            s_row[1] = log2s;
            s_row[2] = rr.gt;
            if (slice == 0 && OP != EPI_LSE_GRAD) {
                if (p.lse_out)
                    p.lse_out[row] = m + kLn2 * log2s;
                if (p.reduction == RED_NONE) {
                    if (p.out)
                        p.out[row] = rr.loss;
                } else {
                    p.partials[row] = (double)rr.loss;
                }
            }
        }
    }
    if constexpr (OP == EPI_NONE) {
        return;
    } else {
        __syncthreads();
        const float m = s_row[0];
        const float log2s = s_row[1];
        const float gt = s_row[2];
        const float mL = m * kLog2e;
        const EpiCoef<DT> ec = epi_coef<DT, EOP>(m, mL, log2s, c);
        const int tail_n = (int)(w.head + p.V - (int64_t)(w.nvec - 1) * E);
        float fx = 0.0f;   // sum of p_j over j != t in this slice (EPI_LSE_GRAD)
        for (int cb = v0; cb < v1; cb += CH) {
            Vec raw[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int v = cb + tid + NT * k;
                raw[k] = ldv(&w.xrow[v < v1 ? v : v1 - 1]);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int v = cb + tid + NT * k;
                if (v < v1) {
                    Vec g = epi_vec<DT, EOP>(raw[k], ec);
                    if (EOP == EPI_GRAD && owner && v == tp.vt)
                        set_elem<DT>(g, tp.jt, gt);
                    store_grad<DT>(w.yrow, v, g, w.head, p.V, p.aligned);
                    if constexpr (OP == EPI_LSE_GRAD) {
                        Vec x = raw[k];
                        if (v == 0 && w.head > 0)
                            mask_outside<DT>(x, w.head, E);
                        if (v == w.nvec - 1)
                            mask_outside<DT>(x, 0, tail_n);
                        if (v == tp.vt)
                            set_elem<DT>(x, tp.jt, -__builtin_inff());
                        fx += vec_sumexp<DT>(x, mL);
                    }
                }
            }
        }
        if constexpr (OP == EPI_LSE_GRAD) {
            __shared__ float s_fx[W];
            const float wf = group_reduce<64>(fx, OpSum());
            if (lane == 0)
                s_fx[wave] = wf;
            __syncthreads();
            if (tid == 0) {
                float f = 0.0f;
#pragma unroll
                for (int i = 0; i < W; ++i)
                    f += s_fx[i];
                p.fix[blockIdx.x] = f;
            }
        }
    }
}

// Backward from a given lse over split rows: where p_t > 1/2, the target's
// gradient is rewritten as -(sum of the other p_j) c from the slices' sums,
// which keeps its relative accuracy.  One wavefront per row.
template <int DT>
__global__ void __launch_bounds__(256) split_fix_kernel(Params p)
{
    constexpr int E = Traits<DT>::E;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= p.M)
        return;
    const int64_t t = row_scalar(p.targets, row);
    const Window w = row_window<DT>(p, row);
    const TargetPos tp = target_pos<DT>(t, p.V, w.head);
    if (!tp.valid)
        return;
    const float lseL = p.lse_in[row] * kLog2e;
    const float pt = fast_exp2(__builtin_fmaf(p.rowx[row], kLog2e, -lseL));
    if (!(pt > 0.5f))
        return;
    const float f = group_reduce<64>(lane < p.S ? p.fix[row * p.S + lane] : 0.0f, OpSum());
    if (lane == 0) {
        Vec g = {};
        set_elem<DT>(g, tp.jt, -f * row_scale(p, row));
        store_partial<DT>(w.yrow + tp.vt, g, tp.jt, tp.jt + 1);
    }
}

}  // namespace cek
