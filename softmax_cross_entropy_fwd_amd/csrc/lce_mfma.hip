// lce_mfma.hip -- the logits of linear + cross-entropy on the matrix cores.
//
// For the lm_head projection z = H W^T ("9 Triton kernels in 9 weeks", week
// 8: the projection chunked into the loss), one workgroup computes a tile of
// z^T = W H^T -- 256 vocabulary rows by 256 tokens -- with bf16 MFMA
// instructions (v_mfma_f32_32x32x16_bf16, fp32 accumulation), and folds it in
// the same kernel:
//
//   stats_kernel  the forward: for every token and every 128 vocabulary rows
//                 of the tile, the (max, sum of exp(z - max)) of the logits
//                 with the target's left out, and the target's logit; the
//                 fp32 logits are never written.  The row combine (finish
//                 kernel) turns these into the loss, the lse and the target's
//                 gradient.
//   grad_kernel   the backward: the gradient g = exp(z - lse) c (the target
//                 taking the gradient the combine computed), rounded to bf16
//                 and written as G [tokens][vocabulary rows of the chunk],
//                 for the dH and dW products.
//
// Data path: A = W rows (vocabulary), B = H rows (tokens), both K-major (the
// nn.Linear layout).  K runs in stages of 64 through two LDS stages of 64
// KiB: buffer loads write each stage's two 256 x 64 tiles straight into LDS
// (no registers, no LDS store instructions), each lane fetching the 16-byte
// chunk that the bank-conflict-free row swizzle puts at its slot; a stage's
// loads go out as soon as the barrier before the last sub-step of the stage
// two back frees its LDS, a whole stage before they are read.  Four
// wavefronts, one per SIMD, each own 128 x 128 of the tile: 4 x 4 blocks of
// 32 x 32, 256 accumulator registers per lane.  With no second wavefront on
// the SIMD to hide latency, every LDS read and every load is placed between
// MFMAs: each sub-step of 16 in K reads its operands while the previous
// one's 16 MFMAs run.  The forward's grid is persistent (a workgroup per
// CU, tiles one after another, the stages one stream across tiles).
//
// In the output of v_mfma_f32_32x32x16_bf16, lane l holds column l % 32 (a
// token) and rows 8 (r / 4) + 4 (l / 32) + r % 4 (vocabulary rows) of its
// block in register r; operand lane l passes row l % 32 and k 8 (l / 32) ..
// 8 (l / 32) + 7 of A, and the same of B (this layout was checked on the
// device).  So each lane reduces its own token over the registers, and the
// two lanes l and l ^ 32 that share a token combine with one exchange.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ce_device.h"
#include "lce_internal.h"

namespace lce {
namespace {

using cek::kLn2;
using cek::kLog2e;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileV = 256;    // vocabulary rows per workgroup tile
constexpr int kTileT = 256;    // tokens per workgroup tile
constexpr int kStepK = 64;     // K per pipeline stage (32 or 64)
constexpr int kThreads = 256;  // four wavefronts, 2 x 2 over the tile
constexpr int kStages = 2;     // LDS stages: one read, the others in flight
constexpr int kSub = kStepK / 16;                   // MFMA sub-steps per stage
constexpr int kRowBytes = kStepK * 2;               // a tile row's bytes in a stage
constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per row and stage
constexpr int kRowsPerLoad = 64 / kChunks;          // tile rows one 1 KiB load fills
constexpr int kOpBytes = kTileV * kRowBytes;        // one operand's tile in a stage (16 KiB)
constexpr int kStageBytes = 2 * kOpBytes;           // 32 KiB
constexpr int kLdsBytes = kStages * kStageBytes;
// loads per wavefront, operand and stage: 1 KiB each; loads per wavefront
// and stage, both operands
constexpr int kLoadsPerWave = kOpBytes / 1024 / (kThreads / 64);
constexpr int kStageLoads = 2 * kLoadsPerWave;
static_assert(kStepK == 32 || kStepK == 64, "stages of 32 or 64 in K");
static_assert(kStages >= 2 && kLdsBytes <= 160 * 1024, "the stages fit the LDS");
constexpr float kNegInf = -__builtin_inff();

// The workgroup's LDS, addressed by offset from the array itself so that
// every access is known to be an LDS access (reached through a generic
// pointer, the operand reads became flat loads, which also wait for the
// global loads in flight).  The stages of both operands.
__shared__ u32x4 g_lds[kLdsBytes / 16];

typedef __attribute__((address_space(3))) void lds_void;

// The tile of virtual block vb.  Blocks are dealt to the eight XCDs in turn
// (block b runs on XCD b % 8, and so does every vb = b + grid j of a
// persistent workgroup when the grid is a multiple of 8); ids are
// renumbered so that each XCD takes a contiguous run of them, and the run
// is walked in groups of kGroup W tiles, W tile fastest, so that the 32
// workgroups an XCD runs at once share 8 W tiles and 4 token tiles in its
// L2.  A bijection for any tile counts.
__device__ __forceinline__ void tile_of(const MfmaParams &q, int vb, int &tv, int &tt)
{
    constexpr int kGroup = 8;
    const int n = q.ntiles_v * q.ntiles_t;
    int id = vb;
    if (n % 8 == 0)
        id = (vb % 8) * (n / 8) + vb / 8;
    const int span = kGroup * q.ntiles_t;   // ids per group of W tiles
    const int g = id / span, r = id % span;
    const int first = g * kGroup;
    const int gv = q.ntiles_v - first < kGroup ? q.ntiles_v - first : kGroup;
    tv = first + r % gv;
    tt = r / gv;
}

// Swizzle of a tile row in a stage: row r's 16-byte chunk c sits at chunk
// c ^ sw(r).  One pass of an operand read serves 16 rows r0 .. r0 + 15
// (r0 % 16 == 0) at one chunk, and their 16-byte slots in the 256 bytes the
// banks serve per cycle must all differ (as must those of any 8 rows in 128
// bytes): with 64-byte rows (4 chunks) a slot is (r % 4, c ^ sw(r)) and
// sw(r) = ((r >> 2) ^ (r >> 1)) & 3; with 128-byte rows (8 chunks) it is
// (r % 2, c ^ sw(r)) and sw(r) = (r & 7) ^ ((r >> 3) & 1).
__device__ __forceinline__ int row_swz(int r)
{
    if constexpr (kChunks == 4)
        return ((r >> 2) ^ (r >> 1)) & 3;
    else
        return (r & 7) ^ ((r >> 3) & 1);
}

// Buffer loads straight into LDS.  Each load instruction of a wavefront
// fills 1 KiB of LDS, lane l the 16 bytes at l: kRowsPerLoad tile rows,
// lane l holding slot l % kChunks of row l / kChunks -- so it fetches the
// chunk that the swizzle puts there.  A resource per operand tile whose records end
// after the tile's last valid row: rows past it read zeros without a branch;
// a K chunk past D gets an offset past every record and reads zeros too.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kOob = 0x7ffffff0;   // >= every num_records (D <= 2^20)
constexpr int kRsrcWord3 = 0x00020000;

struct Loader {
    int roff[kLoadsPerWave];   // byte offset of this lane's row and chunk at k = 0
    int coff[kLoadsPerWave];   // the chunk's byte offset within the row's step
    int wave;                  // wavefront index (uniform)
};

// The buffer resources of a tile's W rows and H rows.
struct Rsrcs {
    Rsrc w, h;
};

__device__ __forceinline__ Loader make_loader(const MfmaParams &q)
{
    Loader L;
    const int rowbytes = (int)q.D * 2;
    const int lane = threadIdx.x & 63;
    L.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int r = kRowsPerLoad * (kLoadsPerWave * L.wave + i) + lane / kChunks;
        const int c = (lane % kChunks) ^ row_swz(r);
        L.coff[i] = 16 * c;
        L.roff[i] = r * rowbytes + L.coff[i];
    }
    return L;
}

__device__ __forceinline__ Rsrcs tile_rsrcs(const MfmaParams &q, int vb)
{
    int tv, tt;
    tile_of(q, vb, tv, tt);
    const int vbase = tv * kTileV, tbase = tt * kTileT;
    const int vrows = q.vn - vbase < kTileV ? q.vn - vbase : kTileV;
    const int trows = q.M - tbase < kTileT ? (int)(q.M - tbase) : kTileT;
    const int rowbytes = (int)q.D * 2;
    Rsrcs R;
    R.w = __builtin_amdgcn_make_buffer_rsrc((void *)(q.W + (q.v0 + vbase) * q.D), (short)0,
                                            vrows * rowbytes, kRsrcWord3);
    R.h = __builtin_amdgcn_make_buffer_rsrc((void *)(q.H + (int64_t)tbase * q.D), (short)0,
                                            trows * rowbytes, kRsrcWord3);
    return R;
}

// Load i of a stage (both operands): K [k0, k0 + kStepK) into stage st;
// with real false, zeros (no memory read) into that stage.
__device__ __forceinline__ void issue_load(const Rsrcs &R, const Loader &L, int st, int k0, int D,
                                           int i, bool real)
{
    const bool kin = real && 2 * k0 + L.coff[i] < 2 * D;
    const int off = kin ? L.roff[i] + 2 * k0 : kOob;
    char *base = reinterpret_cast<char *>(g_lds) + st * kStageBytes +
                 (kLoadsPerWave * L.wave + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.w, (lds_void *)base, 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.h, (lds_void *)(base + kOpBytes), 16, off, 0, 0, 0);
}

__device__ __forceinline__ void issue_stage(const Rsrcs &R, const Loader &L, int st, int k0, int D,
                                            bool real)
{
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
        issue_load(R, L, st, k0, D, i, real);
}

// Wait until at most N of this wavefront's loads are in flight (its loads of
// a stage land before those issued after them), then the workgroup barrier:
// every wavefront's loads of that stage are in LDS, and every wavefront's
// LDS reads before it are done.  The memory clobber keeps the compiler from
// moving LDS reads above it.
template <int N>
__device__ __forceinline__ void stage_barrier()
{
    static_assert(N == 0 || N == 8 || N == 16 || N == 24 || N == 32 || N == 48,
                  "a whole number of stages");
    if constexpr (N == 48)
        asm volatile("s_waitcnt vmcnt(48) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 32)
        asm volatile("s_waitcnt vmcnt(32) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 24)
        asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 16)
        asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 8)
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A K sub-step's operands (16 of a stage's kStepK): A rows 128 wv + 32 i + l % 32
// and B rows 128 wt + 32 i + l % 32, chunk 2 s + l / 32.
struct Frags {
    bf16x8 a[4], b[4];
};

// Operand j of sub-step s of stage st (A block j / 2 for even j, B block
// j / 2 for odd j: the first MFMAs' operands first).  Rows differ from the
// lane's row l % 32 by multiples of 32, so the swizzle is the lane's own.
__device__ __forceinline__ void read_frag(Frags &f, int st, int s, int j)
{
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int orow = lane & 31;
    const int ch = (2 * s + (lane >> 5)) ^ row_swz(orow);
    const int i = j >> 1;
    const int row = (j & 1) ? 128 * (wave & 1) + 32 * i + orow : 128 * (wave >> 1) + 32 * i + orow;
    const int byte = st * kStageBytes + ((j & 1) ? kOpBytes : 0) + row * kRowBytes + 16 * ch;
    const bf16x8 v = __builtin_bit_cast(bf16x8, g_lds[byte >> 4]);
    if (j & 1)
        f.b[i] = v;
    else
        f.a[i] = v;
}

__device__ __forceinline__ void read_frags(Frags &f, int st, int s)
{
#pragma unroll
    for (int j = 0; j < 8; ++j)
        read_frag(f, st, s, j);
}

// One sub-step: 16 MFMAs on cur, each followed by a fixed share of the
// other work, the order pinned (sched_barrier) so that no MFMA waits behind
// it: READ, 8 operand reads (sub-step rs of stage rst) in the first 8
// slots; ISSUE, the kStageLoads loads of stage ist, spread over the slots
// after the reads.
template <bool READ, bool ISSUE>
__device__ __forceinline__ void sub_step(f32x16 (&acc)[4][4], const Frags &cur, Frags &nxt, int rst,
                                         int rs, const Rsrcs &R, const Loader &L, int ist, int ik0,
                                         int D, bool real)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[i >> 2], cur.b[i & 3],
                                                                     acc[i >> 2][i & 3], 0, 0, 0);
        if constexpr (READ)
            if (i < 8)
                read_frag(nxt, rst, rs, i);
        if constexpr (ISSUE) {
            // kLoadsPerWave issue_load calls (two loads each) in slots
            // 16 - kLoadsPerWave .. 15
            constexpr int first = 16 - kLoadsPerWave;
            if (i >= first)
                issue_load(R, L, ist, ik0, D, i - first, real);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The tiles of this workgroup: virtual blocks vb = blockIdx.x + gridDim.x j
// (a persistent grid takes several), each the product over all of K --
// acc[vb][tb] is block (vb, tb) of the wavefront's 128 x 128 (vocabulary x
// tokens) -- handed to epi(acc, tv, tt).  The K stages of all the tiles are
// one stream through the kStages LDS stages, across tile boundaries, so a
// tile's first stages load during the last one's epilogue.  Stage g runs
// kSub sub-steps, sub-step s on one register set while sub-step s + 1's
// operands are read into the other; before the last sub-step comes the
// barrier after stage g + 1's loads (stages g + 2 .. g + kStages - 1 may
// stay in flight), which also frees stage g's LDS: the last sub-step reads
// stage g + 1's first operands and sends stage g + kStages's loads into it.
// Past the last stage the loads still go out, reading nothing and writing
// zeros into the freed stage, and the reads take values no MFMA uses: every
// stage runs the same code and the same wait.  PERSIST false: one tile per
// workgroup (the grid covers the tiles), and epi may use the LDS after
// stage_barrier<0>.
template <bool PERSIST, class Epi>
__device__ __forceinline__ void run_tiles(const MfmaParams &q, Epi &&epi)
{
    const int n = q.ntiles_v * q.ntiles_t;
    const int b = (int)blockIdx.x, G = (int)gridDim.x;
    if (b >= n)
        return;
    const int J = PERSIST ? (n - b + G - 1) / G : 1;
    const int D = (int)q.D;
    const int nk = (D + kStepK - 1) / kStepK;
    const int T = J * nk;
    const Loader L = make_loader(q);

    // the issue stream: next stage gi, tile ij, K step ikt, LDS stage ist
    int gi = 0, ij = 0, ikt = 0, ist = 0;
    Rsrcs R = tile_rsrcs(q, b);
    auto advance = [&]() {
        ++gi;
        ist = ist + 1 == kStages ? 0 : ist + 1;
        if (++ikt == nk) {
            ikt = 0;
            if (++ij < J)
                R = tile_rsrcs(q, b + G * ij);
        }
    };
    for (int s = 0; s < kStages; ++s) {
        issue_stage(R, L, ist, ikt * kStepK, D, gi < T);
        advance();
    }
    // stage 0 landed; the kStages - 1 after it may stay in flight
    stage_barrier<(kStages - 1) * kStageLoads>();
    Frags f0, f1;
    read_frags(f0, 0, 0);

    int st = 0;
    for (int j = 0; j < J; ++j) {
        f32x16 acc[4][4];
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[vb][tb][r] = 0.0f;
        for (int kt = 0; kt < nk; ++kt) {
            sub_step<true, false>(acc, f0, f1, st, 1, R, L, 0, 0, D, false);
            if constexpr (kSub == 4) {
                sub_step<true, false>(acc, f1, f0, st, 2, R, L, 0, 0, D, false);
                sub_step<true, false>(acc, f0, f1, st, 3, R, L, 0, 0, D, false);
            }
            const int st_next = st + 1 == kStages ? 0 : st + 1;
            stage_barrier<(kStages - 2) * kStageLoads>();
            // ist == st here: the stream is kStages stages ahead
            sub_step<true, true>(acc, f1, f0, st_next, 0, R, L, st, ikt * kStepK, D, gi < T);
            advance();
            st = st_next;
        }
        int tv, tt;
        tile_of(q, b + G * j, tv, tt);
        epi(acc, tv, tt);
    }
}

// Row (vocabulary index within the wavefront's 128 rows) of register r.
__device__ __forceinline__ int vrow(int vb, int r, int lane)
{
    return 32 * vb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// The forward's fold of a tile (see the file comment).
__device__ __forceinline__ void stats_epilogue(const MfmaParams &q, f32x16 (&acc)[4][4], int tv, int tt)
{
    const int vbase = tv * kTileV, tbase = tt * kTileT;
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int wv = wave >> 1, wt = wave & 1;
    const int v0w = vbase + 128 * wv;         // first vocabulary row of the wavefront (chunk-local)
    const int half = q.half0 + 2 * tv + wv;   // the statistics entry this wavefront writes
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int64_t tok = tbase + 128 * wt + 32 * tb + (lane & 31);
        const bool tin = tok < q.M;
        // the target's index among the wavefront's rows, or -1
        int tl = -1;
        if (tin) {
            const int64_t g = cek::row_scalar(q.targets, tok) - q.v0 - v0w;
            tl = (g >= 0 && g < 128) ? (int)g : -1;
        }
        float m = kNegInf, xt = 0.0f;
        bool have = false;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int v = vrow(vb, r, lane);
                const float z = acc[vb][tb][r];
                if (v == tl) {
                    xt = z;
                    have = true;
                }
                const bool ok = v0w + v < q.vn && v != tl;
                m = ok ? fmaxf(m, z) : m;
            }
        const float mL = m == kNegInf ? 0.0f : m * kLog2e;
        float s = 0.0f;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int v = vrow(vb, r, lane);
                const float e = cek::fast_exp2(__builtin_fmaf(acc[vb][tb][r], kLog2e, -mL));
                s += (v0w + v < q.vn && v != tl) ? e : 0.0f;
            }
        // the partner lane (l ^ 32) holds the token's other rows
        const float m2 = __shfl_xor(m, 32, 64);
        const float s2 = __shfl_xor(s, 32, 64);
        const float M = fmaxf(m, m2);
        const float S = cek::rescale_to(s, m, M) + cek::rescale_to(s2, m2, M);
        if (tin && lane < 32) {
            float *st = q.stats + 2 * (tok * q.nhalf + half);
            st[0] = M;
            st[1] = S;
        }
        if (tin && have)
            q.rowx[tok] = xt;
    }
}

// The forward: a persistent grid (a workgroup per CU), tiles one after
// another.
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
stats_kernel(MfmaParams q)
{
    run_tiles<true>(q, [&](f32x16 (&acc)[4][4], int tv, int tt) { stats_epilogue(q, acc, tv, tt); });
}

// The backward's tile of G = exp(z - lse) c (the target taking the gradient
// the combine computed), rounded to bf16, written as G [tokens][ldg] from
// the accumulators: a lane's registers 4 g .. 4 g + 3 of a block are 4
// consecutive vocabulary rows of its token, one 8-byte store.
__device__ __forceinline__ void grad_epilogue(const MfmaParams &q, f32x16 (&acc)[4][4], int tv, int tt)
{
    const int vbase = tv * kTileV, tbase = tt * kTileT;
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int wv = wave >> 1, wt = wave & 1;
    const int v0w = vbase + 128 * wv;   // first vocabulary row of the wavefront (chunk-local)
    const float l2c = __log2f(q.c);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int64_t tok = tbase + 128 * wt + 32 * tb + (lane & 31);
        if (tok >= q.M)
            continue;
        // exp(z - lse) c = 2^(z log2 e - (lse log2 e - log2 c)), c > 0
        const float bias = q.lse[tok] * kLog2e - l2c;
        const float gt = q.gt[tok];
        const int64_t g = cek::row_scalar(q.targets, tok) - q.v0 - v0w;
        const int tl = (g >= 0 && g < 128) ? (int)g : -1;
        uint16_t *grow = q.G + tok * q.ldg + v0w;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                float e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * gi + j;
                    const float x = cek::fast_exp2(__builtin_fmaf(acc[vb][tb][r], kLog2e, -bias));
                    e[j] = vrow(vb, r, lane) == tl ? gt : x;
                }
                const int v = vrow(vb, 4 * gi, lane);   // the first of the 4 rows
                const uint32_t lo = cek::pack2<cek::DT_BF16>(e[0], e[1]);
                const uint32_t hi = cek::pack2<cek::DT_BF16>(e[2], e[3]);
                if (v0w + v + 4 <= q.vn) {
                    *reinterpret_cast<uint2 *>(grow + v) = make_uint2(lo, hi);
                } else {
                    const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                           (uint16_t)(hi >> 16)};
                    for (int j = 0; j < 4 && v0w + v + j < q.vn; ++j)
                        grow[v + j] = h[j];
                }
            }
    }
}

// The backward: a persistent grid like the forward's.
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
grad_kernel(MfmaParams q)
{
    run_tiles<true>(q, [&](f32x16 (&acc)[4][4], int tv, int tt) { grad_epilogue(q, acc, tv, tt); });
}

}  // namespace

const void *mfma_stats_kernel_fn() { return (const void *)&stats_kernel; }
const void *mfma_grad_kernel_fn() { return (const void *)&grad_kernel; }

}  // namespace lce
