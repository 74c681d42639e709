// ce_api.hip -- the C ABI: argument checks, launch plan, launch.
//
// Every argument check happens before the first HIP call, so a bad call
// returns its status without touching the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <unordered_map>
#include <utility>

#include "ce.h"
#include "ce_device.h"
#include "ce_internal.h"

namespace {

using cek::KernelRef;

constexpr size_t kPartialBytes = sizeof(double) * cek::kMaxPartials;
constexpr int kMaxSplit = 64;            // slices per row
constexpr int64_t kSplitMaxRows = 128;         // rows up to which splitting pays
constexpr int64_t kSplitMaxRowsForced = 512;   // bound of the workspace's split scratch
constexpr int64_t kSplitMinVecs = 16384;       // 256 KiB rows
constexpr size_t kSplitBytesPerSlice = 12;   // (max, sum) + the target-fix sum, fp32

size_t elem_size(int dtype) { return dtype == CE_F32 ? 4 : 2; }

struct Plan {
    int split = 0, slice_vecs = 0;   // slices per row (0: one workgroup or group per row)
    int kind = 0, a = 0, b = 0;
    bool exact = false;
    int nbuf = 1;
    KernelRef k{nullptr, 0};
    int64_t grid = 0;
    int units_per_wg = 1;   // partial sums each workgroup publishes
    int occupancy = 0;
    int cus = 0;
    bool blocked = false;   // each workgroup walks a contiguous band of rows
};

KernelRef lookup(int dtype, int op, int kind, int a, int b, bool exact, int nbuf)
{
    using Fn = KernelRef (*)(int, int, int, int, bool, int);
    static const Fn table[3][3] = {
        {cek::get_kernel_f32_fwd, cek::get_kernel_f32_grad, cek::get_kernel_f32_aux},
        {cek::get_kernel_f16_fwd, cek::get_kernel_f16_grad, cek::get_kernel_f16_aux},
        {cek::get_kernel_bf16_fwd, cek::get_kernel_bf16_grad, cek::get_kernel_bf16_aux},
    };
    const int part = op == cek::EPI_NONE ? 0 : op == cek::EPI_GRAD ? 1 : 2;
    return table[dtype][part](op, kind, a, b, exact, nbuf);
}

cek::SplitKernels split_kernels(int dtype)
{
    return dtype == CE_F32 ? cek::split_kernels_f32()
           : dtype == CE_F16 ? cek::split_kernels_f16()
                             : cek::split_kernels_bf16();
}

// Vectors one tile of a shape covers (0 for the stream kernels: any row).
int64_t tile_vectors(int kind, int a, int b)
{
    if (kind == cek::KIND_ROWS)
        return (int64_t)a * b;
    if (kind == cek::KIND_WG || kind == cek::KIND_WG2)
        return (int64_t)a * 64 * b;
    return 0;
}

int pow2ceil(int64_t n)
{
    int p = 1;
    while (p < n)
        p <<= 1;
    return p;
}

// Mapping and tile for a row of nvec 16-byte vectors (worst case over rows),
// from measurements on MI355X:
//  - the forward of rows of 257-1536 vectors (4-24 KB; fp32 rows from 129
//    vectors) streams each row
//    through one wavefront in chunks of 64 K vectors (K = 8 up to 512
//    vectors, then 4), 8 wavefronts per CU for fp32 rows and 12 for 16-bit
//    ones.  Against the rows kernel's register tiles (region times, ~530 MB
//    of logits): fp32 1500 wide 91 / 113 us, 2000 wide 80 / 85, 3000 wide
//    118 / 176, 4000 wide 98 / 113, 4096 wide 82.4 / 83.2; bf16 4000 wide
//    88 / 91, 6000 wide 98 / 131, 8000 wide 84 / 95, 8192 wide 86 / 89: a
//    tile the row does not fill still takes a full tile's time;
//  - shorter rows sit in the registers of 1..64 lanes (rows kernel), and so
//    do the rows of the epilogues up to 16 KB;
//  - longer rows are streamed for the forward by 4-, 8- or 16-wave
//    workgroups as the rows grow;
//  - the epilogues (fused backward, softmax, ...) past 16 KB: rows whose
//    re-read stays in L2 while the CU's other rows stream are streamed
//    twice (up to 48 KB by 8-wave workgroups, 32 waves per CU; up to 128 KB
//    by one 16-wave workgroup per CU), unless they fill a 16-wave register
//    tile exactly; rows of 128-256 KB sit in the registers of a 16-wave
//    workgroup (one HBM read per element), longer ones are streamed again.
//    A register tile that the row leaves partly empty costs nearly as much
//    as a full one: the workgroup waits out each row's loads, so the tile,
//    not the data, sets the time.
// 16-bit rows of 4097-6656 vectors that do not fill a 16-wave tile exactly
// sit in 8-wave register tiles, two workgroups per CU, so that one row's
// reduction overlaps the other's memory traffic.
// *waves: waves per CU the grid is sized for (0: the mapping's default).
void choose_shape(int64_t nvec, bool bwd, bool aligned, bool wide, int *kind, int *a, int *b,
                  int *nbuf, int *waves)
{
    *nbuf = 1;
    *waves = 0;
    *kind = cek::KIND_ROWS;
    if (!bwd && nvec > 256 && nvec <= 1536) {
        *kind = cek::KIND_WSTREAM;
        *a = 1;
        *b = nvec > 512 ? 4 : 8;
        *waves = wide ? 12 : 8;
    } else if (!bwd && !wide && nvec > 128 && nvec <= 256) {
        // fp32 rows of 129-256 vectors: one chunk per row, more wavefronts
        // the shorter it is (region times against the rows kernel, ~530 MB:
        // 700 wide 94 / 107 us at 16, 800 wide 98 / 110 at 16, 900 wide 73 /
        // 81 at 12, 1000 wide 82 / 86 at 12); 16-bit rows this short stay
        // in register rows (1800 wide 99 / 92)
        *kind = cek::KIND_WSTREAM;
        *a = 1;
        *b = 4;
        *waves = nvec > 208 ? 12 : 16;
    } else if (nvec <= 4) {
        *a = 1;
        *b = nvec <= 1 ? 1 : nvec <= 2 ? 2 : 4;
    } else if (nvec <= 8) {
        *a = 2;
        *b = 4;
    } else if (nvec <= 16) {
        *a = 4;
        *b = 4;
    } else if (nvec <= 32 && !bwd) {
        // 8 lanes per row: whole 128-byte lines per load instruction, so the
        // loads can be non-temporal and the target's logit is taken from the
        // registers (fp32 1M x 128 forward 87 us against 90-104 us, box to
        // box, with 4 lanes x 8 vectors and two register sets; bf16 1M x 256
        // 92 against 125)
        *a = 8;
        *b = 4;
    } else if (nvec <= 32) {
        *a = 4;
        *b = 8;
        *nbuf = 2;
    } else if (nvec <= 256) {
        // rows of 33-256 vectors (the fp32 forwards of 129-256 stream, above):
        // the power-of-two lanes per row that leave 4-6 vectors per lane, so
        // the tile fits the row (the fold and the epilogue run over every
        // slot of a tile).  Measured per launch (1M rows unless noted), 4
        // vectors per lane against the fitted tile: forwards fp32 160 wide
        // 138 / 109 us (8 x 5), misaligned f16 250 wide 224 / 137, fp32 320
        // wide (512K rows) 143 / 105 (16 x 5), bf16 384 wide 180 / 136 (8 x
        // 6); fused backward f16 250 wide 367 / 322, bf16 384 wide 331 / 305,
        // bf16 1200 wide (256K rows) 322 / 246 (32 x 5), fp32 320 wide 257 /
        // 248; bf16 384 wide softmax 314 / 291.  fp32 epilogues of 129-256
        // vectors keep 64 x 4 (600 wide: softmax 254 / 260, fused backward
        // 241 / 240 in 32 x 5).
        const int g = nvec <= 48 ? 8 : nvec <= 96 ? 16 : nvec <= 128 ? 32
                      : (wide && nvec <= 192) ? 32 : 64;
        *a = g;
        *b = g == 64 ? 4 : (int)((nvec + g - 1) / g);
    } else if (nvec <= 512) {
        *a = 64;
        *b = 8;
    } else if (nvec <= 1024) {
        *a = 64;
        *b = 16;
    } else if (bwd && nvec <= 8192 && aligned && nvec % 1024 == 0 && nvec > 3072) {
        // an exact 16-wave register tile
        *kind = cek::KIND_WG;
        *a = 16;
        *b = (int)(nvec / 1024);
    } else if (bwd && nvec <= 3072) {
        // measured (fused fwd+bwd, 1 GiB of logits): 1500 vectors 464 us
        // against 1036 with a 4096-vector register tile; 3072: 452 against 490
        // in an exact 3072 tile
        *kind = cek::KIND_STREAM;
        *a = 8;
        *b = 4;
        *waves = 32;
    } else if (bwd && wide && nvec > 4096 && nvec <= 6656) {
        // measured (fused fwd+bwd, 1 GiB of bf16 logits, us): 4500 vectors
        // 445 against 488 streamed; 5000: 418 / 494; 6000: 424 / 457; the
        // stress rows 354 / 360; at 7000 the two tie, at 7500 streaming wins
        *kind = cek::KIND_WG2;
        *a = 8;
        *b = (int)((nvec + 511) / 512);
        *waves = 16;
    } else if (bwd && nvec <= 8192) {
        // measured: the stress rows (6283 vectors, fp16) 358 us against 394
        // in an 8192 tile and 371 in a 7168 one; fp32 6000 vectors 484
        // against 662 (8192) and 643 (6144)
        *kind = cek::KIND_STREAM;
        *a = 16;
        *b = 4;
    } else if (bwd && nvec <= 16384) {
        *kind = cek::KIND_WG;
        *a = 16;
        *b = nvec <= 12288 ? 12 : 16;
    } else {
        // chunks of W*64*4 vectors; more, smaller workgroups per CU until the
        // rows are long enough to keep a wide one busy (measured: 6283
        // vectors 5.2 TB/s with W=4 against 4.7 with W=8; 15000 vectors 5.6
        // with W=16 against 5.4 with W=8)
        *kind = cek::KIND_STREAM;
        *a = nvec >= 14336 ? 16 : (!bwd && nvec < 8192) ? 4 : 8;
        *b = 4;
    }
}

// CE_FORCE_PLAN=rows:G:K | wg:W:K | wg2:W:K | stream:W:K | wstream:1:K overrides the
// mapping (tuning).
bool parse_forced_shape(const char *s, int *kind, int *a, int *b)
{
    if (!s || !*s)
        return false;
    char name[16] = {0};
    int x = 0, y = 0;
    if (std::sscanf(s, "%15[a-z0-9]:%d:%d", name, &x, &y) != 3)
        return false;
    if (!std::strcmp(name, "rows"))
        *kind = cek::KIND_ROWS;
    else if (!std::strcmp(name, "wg"))
        *kind = cek::KIND_WG;
    else if (!std::strcmp(name, "stream"))
        *kind = cek::KIND_STREAM;
    else if (!std::strcmp(name, "wstream"))
        *kind = cek::KIND_WSTREAM;
    else if (!std::strcmp(name, "wg2"))
        *kind = cek::KIND_WG2;
    else
        return false;
    *a = x;
    *b = y;
    return true;
}

// The tuning environment variables, read once (at the first call, and again
// by ce_tuning_reload): CE_FORCE_PLAN, CE_FORCE_SPLIT, CE_FORCE_NBUF,
// CE_WAVES_PER_CU, CE_FORCE_GRID, CE_ROW_MAP, CE_LINEAR_GEMM and
// CE_FUSE_MAX_BYTES.
// `generation` changes on every reload, so cached plans follow.
struct Tuning {
    bool plan_set = false;       // CE_FORCE_PLAN non-empty
    bool plan_ok = false;        // ... and parsed
    int fk = 0, fa = 0, fb = 0;  // its shape
    int force_split = -1;        // CE_FORCE_SPLIT (-1: unset)
    int force_nbuf = 0;          // CE_FORCE_NBUF (0: unset)
    int waves_per_cu = 0;        // CE_WAVES_PER_CU (0: unset)
    int64_t force_grid = 0;      // CE_FORCE_GRID (0: unset)
    int row_map = 0;             // CE_ROW_MAP: 0 unset, 1 interleaved, 2 blocked
    bool linear_library = false; // CE_LINEAR_GEMM=library
    int64_t fuse_max_bytes = -1; // CE_FUSE_MAX_BYTES (-1: unset)
    unsigned generation = 0;
};

Tuning g_tuning;
std::once_flag g_tuning_once;
std::mutex g_tuning_mu;

void read_tuning(Tuning *t)
{
    const unsigned gen = t->generation + 1;
    *t = Tuning();
    t->generation = gen;
    const char *fp = std::getenv("CE_FORCE_PLAN");
    t->plan_set = fp && *fp;
    t->plan_ok = parse_forced_shape(fp, &t->fk, &t->fa, &t->fb);
    const char *f = std::getenv("CE_FORCE_SPLIT");
    t->force_split = (f && *f) ? std::atoi(f) : -1;
    const char *nb = std::getenv("CE_FORCE_NBUF");
    t->force_nbuf = nb ? std::atoi(nb) : 0;
    const char *tw = std::getenv("CE_WAVES_PER_CU");
    t->waves_per_cu = (tw && std::atoi(tw) > 0) ? std::atoi(tw) : 0;
    const char *g = std::getenv("CE_FORCE_GRID");
    t->force_grid = (g && *g && std::atoll(g) > 0) ? std::atoll(g) : 0;
    const char *map = std::getenv("CE_ROW_MAP");
    t->row_map = !map                                ? 0
                 : !std::strcmp(map, "blocked")      ? 2
                 : !std::strcmp(map, "interleaved")  ? 1
                                                     : 0;
    const char *lg = std::getenv("CE_LINEAR_GEMM");
    t->linear_library = lg && !std::strcmp(lg, "library");
    const char *fm = std::getenv("CE_FUSE_MAX_BYTES");
    t->fuse_max_bytes = (fm && *fm) ? std::atoll(fm) : -1;
}

const Tuning &tuning()
{
    std::call_once(g_tuning_once, [] { read_tuning(&g_tuning); });
    return g_tuning;
}

bool forced_shape(int *kind, int *a, int *b)
{
    const Tuning &t = tuning();
    if (!t.plan_ok)
        return false;
    *kind = t.fk;
    *a = t.fa;
    *b = t.fb;
    return true;
}

std::mutex g_mu;
std::unordered_map<int, int> g_cus;                       // device -> CU count
std::unordered_map<uint64_t, int> g_occ;                  // (device, fn) -> blocks per CU

int device_cus(int dev, int *cus)
{
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) {
        *cus = it->second;
        return CE_OK;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return CE_ERR_HIP;
    g_cus[dev] = n;
    *cus = n;
    return CE_OK;
}

int blocks_per_cu(int dev, const KernelRef &k, int *occ)
{
    uint64_t key = ((uint64_t)(uint32_t)dev << 48) ^ (uint64_t)(uintptr_t)k.fn;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) {
        *occ = it->second;
        return CE_OK;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k.fn, k.block, 0) != hipSuccess)
        return CE_ERR_HIP;
    if (n < 1)
        n = 1;
    g_occ[key] = n;
    *occ = n;
    return CE_OK;
}

// Worst-case 16-byte vectors a row window spans.
int64_t window_vectors(int64_t V, int E, bool aligned)
{
    return aligned ? V / E : (V + 2 * E - 2) / E;
}

// Slices per row when the rows are long and too few to fill the device one
// workgroup per row (0: no split): about 1024 workgroups in all, slices of
// whole chunks.  Measured on MI355X: splitting pays for at most 128 rows of
// at least 256 KiB (a 2 MiB bf16 row: 112 -> 23 us for the fused backward),
// and loses to the one-row kernels from about 256 rows on.
// CE_FORCE_SPLIT=S forces S slices for up to 512 rows of 32 KiB and more
// (0 disables splitting); CE_FORCE_PLAN disables it unless CE_FORCE_SPLIT is
// set.  Both are for tuning and tests.
int split_slices(int64_t M, int64_t nvec, int *slice_vecs)
{
    const Tuning &t = tuning();
    const int forced = t.force_split;
    if (forced == 0 || (forced < 0 && t.plan_set))
        return 0;
    const int64_t max_rows = forced > 0 ? kSplitMaxRowsForced : kSplitMaxRows;
    const int64_t min_vecs = forced > 0 ? 2 * cek::kSplitChunk : kSplitMinVecs;
    if (M < 1 || M > max_rows || nvec < min_vecs)
        return 0;
    int64_t S = forced > 0 ? forced : (1024 + M - 1) / M;
    const int64_t by_len = nvec / cek::kSplitChunk;
    if (S > by_len)
        S = by_len;
    if (S > kMaxSplit)
        S = kMaxSplit;
    if (S < 2)
        return 0;
    int64_t sv = (nvec + S - 1) / S;
    sv = (sv + cek::kSplitChunk - 1) / cek::kSplitChunk * cek::kSplitChunk;
    S = (nvec + sv - 1) / sv;
    if (S < 2)
        return 0;
    *slice_vecs = (int)sv;
    return (int)S;
}

// Workspace bytes a call uses: the partial-sum slots when it reduces losses,
// then the split scratch when its rows are split.
size_t used_workspace(int64_t M, bool reduced, int S)
{
    if (S > 0)
        return kPartialBytes + (size_t)M * ((size_t)S * kSplitBytesPerSlice + 4);
    return reduced ? kPartialBytes : 0;
}

int make_plan(int64_t M, int64_t V, int dtype, int op, bool aligned, Plan *plan)
{
    const int E = 16 / (int)elem_size(dtype);
    const int64_t nvec = window_vectors(V, E, aligned);
    int kind = 0, a = 0, b = 0, nbuf = 1, waves = 0;
    choose_shape(nvec, op != cek::EPI_NONE, aligned, E == 8, &kind, &a, &b, &nbuf, &waves);
    // The backward from a given lse needs no row in registers: for long
    // 16-bit rows, 8-wave streaming workgroups, as many as fit, beat the
    // register-resident workgroup (measured: LM head 5.24 against 4.98 TB/s,
    // 50257-wide fp16 rows 4.98 against 4.31); fp32 rows stay resident.
    const bool lse_stream = op == cek::EPI_LSE_GRAD && dtype != CE_F32 && nvec >= 4096;
    if (lse_stream) {
        kind = cek::KIND_STREAM;
        a = 8;
        b = 4;
        nbuf = 1;
        waves = 32;
    }
    int fk, fa, fb;
    if (forced_shape(&fk, &fa, &fb)) {
        const int64_t tile = tile_vectors(fk, fa, fb);
        if (lookup(dtype, op, fk, fa, fb, false, 1).fn &&
            (fk == cek::KIND_STREAM || fk == cek::KIND_WSTREAM || tile >= nvec)) {
            kind = fk;
            a = fa;
            b = fb;
            nbuf = 1;
            waves = 0;
        }
    }
    plan->kind = kind;
    plan->a = a;
    plan->b = b;
    plan->exact = aligned && tile_vectors(kind, a, b) == nvec;
    plan->nbuf = kind == cek::KIND_ROWS ? nbuf : 1;
    const int fnb = tuning().force_nbuf;
    if (kind == cek::KIND_ROWS && (fnb == 1 || fnb == 2 || fnb == 17 || fnb == 18))
        plan->nbuf = fnb;
    plan->k = lookup(dtype, op, kind, a, b, plan->exact, plan->nbuf);
    if (!plan->k.fn && plan->nbuf != nbuf) {   // an override with no such instance
        plan->nbuf = kind == cek::KIND_ROWS ? nbuf : 1;
        plan->k = lookup(dtype, op, kind, a, b, plan->exact, plan->nbuf);
    }
    if (!plan->k.fn)
        return CE_ERR_HIP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return CE_ERR_HIP;
    int rc = device_cus(dev, &plan->cus);
    if (rc)
        return rc;
    rc = blocks_per_cu(dev, plan->k, &plan->occupancy);
    if (rc)
        return rc;
    int64_t rows_per_wg = kind == cek::KIND_ROWS      ? (plan->k.block / 64) * (64 / a)
                          : kind == cek::KIND_WSTREAM ? plan->k.block / 64
                                                      : 1;
    int64_t needed = (M + rows_per_wg - 1) / rows_per_wg;
    // Wavefronts per CU.  The rows kernels keep K vectors (K KiB) per
    // wavefront in flight, one row ahead; enough wavefronts to hold about
    // 64 KiB per CU in flight, or 128 KiB where each row is folded before
    // its epilogue (softmax, fused backward) or is 16-bit (twice the VALU
    // work per byte), between 4 and 16.  Measured on MI355X: fp32 4096-wide
    // forward 85.7 us at 4 wavefronts against 89.8 at 8; its softmax 210 ->
    // 200 us at 8; bf16 2000-wide forward 191 -> 100 us at 16; fp32
    // 2000-wide forward 125 -> 90 us at 8.  Two-buffer rows kernels (narrow
    // rows, two rows per lane in flight) keep 4: 8 cost 2-10 %.  The
    // workgroup kernels run 16.
    const int waves_per_wg = plan->k.block / 64;
    const int tw = tuning().waves_per_cu;
    int rows_waves = 4;
    if (kind == cek::KIND_ROWS && plan->nbuf == 1) {
        const bool folded_epilogue =
            op == cek::EPI_GRAD || op == cek::EPI_SOFTMAX || op == cek::EPI_LOGSOFTMAX;
        const int target_kib = (dtype != CE_F32 || folded_epilogue) ? 128 : 64;
        // to the nearest whole number of 4-wave workgroups (fp32 6 vectors
        // per lane: 12 wavefronts, 126 us for 512K x 380 against 137 at 8)
        rows_waves = 4 * ((target_kib + 2 * b) / (4 * b));
        rows_waves = rows_waves < 4 ? 4 : rows_waves > 16 ? 16 : rows_waves;
        // fp32 forwards over 8+ lanes per row (non-temporal loads): 12
        // (per launch at 12 / 16: 1M x 128 84.6 / 85.8 us, 512K x 256 84.6 /
        // 85.9, 256K x 512 83.7 / 86.0; narrower rows and 16-bit ones keep
        // 16: fp32 4M x 20 114 / 97, f16 256K x 1000 99 / 93)
        if (dtype == CE_F32 && op == cek::EPI_NONE && a >= 8 && rows_waves > 12)
            rows_waves = 12;
    }
    const int target_waves = tw > 0                   ? tw
                             : kind == cek::KIND_ROWS ? rows_waves
                             : waves > 0              ? waves
                                                      : 16;
    int wg_per_cu = target_waves / waves_per_wg;
    if (wg_per_cu < 1)
        wg_per_cu = 1;
    if (wg_per_cu > plan->occupancy)
        wg_per_cu = plan->occupancy;
    int64_t cap = (int64_t)plan->cus * wg_per_cu;
    if (tuning().force_grid > 0)
        cap = tuning().force_grid;
    // one published partial per workgroup
    const int64_t units_per_wg = 1;
    plan->units_per_wg = (int)units_per_wg;
    if (cap * units_per_wg > cek::kMaxPartials)
        cap = cek::kMaxPartials / units_per_wg;
    plan->grid = needed < cap ? needed : cap;
    if (plan->grid < 1)
        plan->grid = 1;
    // Row order: the whole grid strides over the rows, or (CE_ROW_MAP=blocked,
    // for tuning) each workgroup walks its own contiguous band.  Bands
    // measured faster only for the 4096-wide fp32 forward in register rows
    // (84.7-85.3 against 85.6-86.2 us), which now streams its rows instead;
    // slower elsewhere (1048576 x 128 fp32 forward +3 %, LM head fused
    // backward +1.4 %, 8 or 16 wavefronts per CU +1 %).
    plan->blocked = false;
    if (tuning().row_map && (kind == cek::KIND_ROWS || kind == cek::KIND_WG || kind == cek::KIND_WG2))
        plan->blocked = tuning().row_map == 2;   // the kernels with a choice of row order
    return CE_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || !na || !nb)
        return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Everything one call hands over.  Pointers a given operation does not use
// are null.
struct Call {
    int op = cek::EPI_NONE;
    const void *logits = nullptr;
    const int64_t *targets = nullptr;
    int64_t M = 0, V = 0;
    int dtype = CE_F32;
    int reduction = CE_NONE;
    float *out = nullptr;          // losses: [M] (none) or [1]
    float *lse_out = nullptr;      // [M] or null
    const float *lse_in = nullptr; // [M] (split backward)
    const float *dloss = nullptr;  // [M] (none) or [1] (split backward), or null
    void *y = nullptr;             // [M, V] epilogue output (may equal logits)
    void *ws = nullptr;
    size_t ws_bytes = 0;
    bool loss = true;              // computes losses (needs targets and out)
    bool own_scratch = false;      // ws is the library's static scratch (ce_fwd_noalloc)
};

struct Region {
    const void *p;
    size_t n;
};

// Slices per row the plan would split this call's rows into given room for
// the split scratch (0: not split), and the workspace bytes that takes.
int planned_split(const Call &c, int *slice_vecs, size_t *bytes)
{
    const bool reduced = c.loss && c.reduction != CE_NONE;
    *bytes = used_workspace(c.M, reduced, 0);
    if (c.M < 1)
        return 0;
    const size_t s = elem_size(c.dtype);
    const int E = 16 / (int)s;
    const int head0 = (int)(((uintptr_t)c.logits % 16) / s);
    const bool aligned = head0 == 0 && c.V % E == 0;
    int sv = 0;
    const int S = split_slices(c.M, window_vectors(c.V, E, aligned), &sv);
    if (S < 2)
        return 0;
    *bytes = used_workspace(c.M, reduced, S);
    if (slice_vecs)
        *slice_vecs = sv;
    return S;
}

// Slices per row this call uses: split rows need the workspace's scratch.
int call_split(const Call &c, int *slice_vecs)
{
    if (c.M < 1 || !c.ws)
        return 0;
    size_t need = 0;
    int sv = 0;
    const int S = planned_split(c, &sv, &need);
    if (S < 2 || c.ws_bytes < need)
        return 0;
    if (slice_vecs)
        *slice_vecs = sv;
    return S;
}

// split: receives the slices per row the call uses (call_split), when the
// arguments pass.
int check_args(const Call &c, int *split = nullptr, int *slice_vecs = nullptr)
{
    if (c.dtype != CE_F32 && c.dtype != CE_F16 && c.dtype != CE_BF16)
        return CE_ERR_DTYPE;
    if (c.reduction != CE_NONE && c.reduction != CE_MEAN && c.reduction != CE_SUM)
        return CE_ERR_REDUCTION;
    if (c.M < 0 || c.V < 1 || c.V > CE_MAX_V)
        return CE_ERR_SHAPE;
    const size_t s = elem_size(c.dtype);
    if (c.M > 0 && (uint64_t)c.M > (uint64_t)INT64_MAX / (uint64_t)c.V / s)
        return CE_ERR_SHAPE;
    const bool reduced = c.loss && c.reduction != CE_NONE;
    if (split)
        *split = 0;
    if (c.M == 0) {
        if (reduced && !c.out)
            return CE_ERR_NULL;
        return CE_OK;
    }
    const bool needs_targets = c.loss || c.op == cek::EPI_LSE_GRAD;
    const bool has_y = c.op != cek::EPI_NONE;
    if (!c.logits || (needs_targets && !c.targets) || (c.loss && !c.out) || (has_y && !c.y) ||
        (c.op == cek::EPI_LSE_GRAD && !c.lse_in))
        return CE_ERR_NULL;
    if ((uintptr_t)c.logits % s || (uintptr_t)c.targets % 8 || (uintptr_t)c.out % 4 ||
        (uintptr_t)c.lse_out % 4 || (uintptr_t)c.lse_in % 4 || (uintptr_t)c.dloss % 4)
        return CE_ERR_ALIGNMENT;
    // the output is written with the vectors the input is read with
    if (has_y && (uintptr_t)c.y % 16 != (uintptr_t)c.logits % 16)
        return CE_ERR_ALIGNMENT;
    // (the library's own scratch is sized and placed by ce_fwd_noalloc)
    if (reduced && !c.own_scratch) {
        if (!c.ws || c.ws_bytes < kPartialBytes || (uintptr_t)c.ws % 8)
            return CE_ERR_WORKSPACE;
    }
    if (c.ws && (uintptr_t)c.ws % 8)
        return CE_ERR_WORKSPACE;
    // Outputs may not overlap one another or any input; the epilogue output
    // may be the logits themselves (exactly, in place).
    const size_t xb = (size_t)c.M * (size_t)c.V * s;
    const size_t per_row = (size_t)c.M * 4;
    const size_t nd = c.reduction == CE_NONE ? per_row : 4;
    int sv = 0;
    const int S = call_split(c, &sv);
    const Region outs[] = {
        {c.out, c.loss ? (c.reduction == CE_NONE ? per_row : 4) : 0},
        {c.lse_out, per_row},
        {c.y == c.logits ? nullptr : c.y, has_y ? xb : 0},
        {c.y == c.logits ? c.y : nullptr, has_y ? xb : 0},
        // a static device symbol of the library cannot overlap the caller's buffers
        {c.own_scratch ? nullptr : c.ws, used_workspace(c.M, reduced, S)},
    };
    const Region ins[] = {
        {c.y == c.logits ? nullptr : c.logits, xb},
        {c.targets, needs_targets ? (size_t)c.M * 8 : 0},
        {c.lse_in, c.op == cek::EPI_LSE_GRAD ? per_row : 0},
        {c.dloss, c.op == cek::EPI_LSE_GRAD ? nd : 0},
    };
    const int no = sizeof(outs) / sizeof(outs[0]), ni = sizeof(ins) / sizeof(ins[0]);
    for (int i = 0; i < no; ++i) {
        for (int j = i + 1; j < no; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return CE_ERR_ALIAS;
        for (int j = 0; j < ni; ++j)
            if (overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n))
                return CE_ERR_ALIAS;
    }
    if (split)
        *split = S;
    if (slice_vecs)
        *slice_vecs = sv;
    return CE_OK;
}

// Plans of recent calls, per host thread: a call repeats the last few
// shapes far more often than not, and a hit skips make_plan's device
// queries.  Keyed by everything make_plan reads, the tuning generation
// included.
struct PlanKey {
    int64_t M = -1, V = 0;
    int dtype = 0, op = 0, dev = -1;
    bool aligned = false;
    unsigned gen = 0;
    bool operator==(const PlanKey &o) const
    {
        return M == o.M && V == o.V && dtype == o.dtype && op == o.op && dev == o.dev &&
               aligned == o.aligned && gen == o.gen;
    }
};
constexpr int kPlanCache = 8;
thread_local PlanKey t_plan_keys[kPlanCache];
thread_local Plan t_plans[kPlanCache];
thread_local int t_plan_next = 0;

int cached_plan(int64_t M, int64_t V, int dtype, int op, bool aligned, Plan *plan)
{
    PlanKey key;
    key.M = M;
    key.V = V;
    key.dtype = dtype;
    key.op = op;
    key.aligned = aligned;
    key.gen = tuning().generation;
    if (hipGetDevice(&key.dev) != hipSuccess)
        return CE_ERR_HIP;
    for (int i = 0; i < kPlanCache; ++i)
        if (t_plan_keys[i] == key) {
            *plan = t_plans[i];
            return CE_OK;
        }
    const int rc = make_plan(M, V, dtype, op, aligned, plan);
    if (rc)
        return rc;
    t_plan_keys[t_plan_next] = key;
    t_plans[t_plan_next] = *plan;
    t_plan_next = (t_plan_next + 1) % kPlanCache;
    return CE_OK;
}

// ---- the final sum in the kernel's own launch (finish_in_kernel) ----------
// A mean or sum over whole rows finishes in the launch that made the
// partials, which saves the second launch and the gap before it (measured
// on MI355X: 1 to 2 us at every size, 87.3 -> 86.3 us for 32768 x 4096
// fp32).  Each (device, stream) gets a counter in the library's device
// memory (zero at load, and put back to zero by every launch that uses it);
// calls on one stream run in order, so they never share a counter at the
// same time.  Calls being captured into a graph, split rows, and streams
// past the last counter keep the second launch.  CE_FUSE_MAX_BYTES=N limits
// the fused form to inputs of at most N bytes (0: never; tuning and tests).
constexpr int kTicketSlots = 1024;
constexpr int kMaxTicketDevices = 64;

}  // namespace

static __device__ unsigned tickets[kTicketSlots];

namespace {

std::mutex g_ticket_mu;
unsigned *g_ticket_base[kMaxTicketDevices];
std::map<std::pair<int, hipStream_t>, int> g_ticket_slot;
thread_local int t_ticket_dev = -1;
thread_local hipStream_t t_ticket_stream = nullptr;
thread_local unsigned *t_ticket = nullptr;

// The counter of (current device, st), or null (second launch instead).
unsigned *ticket_for(hipStream_t st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxTicketDevices)
        return nullptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return nullptr;
    if (t_ticket && t_ticket_dev == dev && t_ticket_stream == st)
        return t_ticket;
    std::lock_guard<std::mutex> lk(g_ticket_mu);
    if (!g_ticket_base[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(tickets)) != hipSuccess || !p)
            return nullptr;
        g_ticket_base[dev] = (unsigned *)p;
    }
    auto it = g_ticket_slot.find({dev, st});
    int slot;
    if (it != g_ticket_slot.end()) {
        slot = it->second;
    } else {
        slot = 0;
        for (const auto &kv : g_ticket_slot)
            if (kv.first.first == dev)
                ++slot;
        if (slot >= kTicketSlots)
            return nullptr;
        g_ticket_slot[{dev, st}] = slot;
    }
    t_ticket_dev = dev;
    t_ticket_stream = st;
    t_ticket = g_ticket_base[dev] + slot;
    return t_ticket;
}

int run(const Call &c, void *stream)
{
    int S = 0, slice_vecs = 0;
    int rc = check_args(c, &S, &slice_vecs);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    if (c.M == 0) {
        if (!c.loss || c.reduction == CE_NONE)
            return CE_OK;
        float value = c.reduction == CE_MEAN ? __builtin_nanf("") : 0.0f;
        float *out = c.out;
        void *args[] = {&out, &value};
        if (hipLaunchKernel(cek::empty_reduce_fn(), dim3(1), dim3(64), args, 0, st) != hipSuccess)
            return CE_ERR_HIP;
        return CE_OK;
    }
    const size_t s = elem_size(c.dtype);
    const int E = 16 / (int)s;
    const uintptr_t base = (uintptr_t)c.logits;
    const int head0 = (int)((base % 16) / s);
    const bool aligned = head0 == 0 && c.V % E == 0;
    Plan plan;
    if (S == 0) {
        rc = cached_plan(c.M, c.V, c.dtype, c.op, aligned, &plan);
        if (rc)
            return rc;
    }

    const int reduction = c.loss ? c.reduction : CE_NONE;
    cek::Params p;
    p.x = (cek::Vec *)(base - (uintptr_t)head0 * s);
    p.y = c.y ? (cek::Vec *)((uintptr_t)c.y - (uintptr_t)head0 * s) : nullptr;
    p.targets = c.targets;
    p.out = c.loss ? c.out : nullptr;
    p.partials = reduction == CE_NONE ? nullptr : (double *)c.ws;
    p.M = c.M;
    p.V = c.V;
    p.head0 = head0;
    p.aligned = aligned ? 1 : 0;
    p.blocked = plan.blocked ? 1 : 0;
    // Only calls that compute losses reduce them (and have a workspace); the
    // split backward uses its reduction for the gradient scale and the shape
    // of dloss alone.
    p.reduction = reduction;
    if (reduction != CE_NONE && !p.partials)
        return CE_ERR_WORKSPACE;
    const double scale = c.reduction == CE_MEAN ? 1.0 / (double)c.M : 1.0;
    p.c = (float)scale;
    p.out_scale = scale;
    p.dloss = c.dloss;
    p.dloss_per_row = c.reduction == CE_NONE ? 1 : 0;
    p.lse_out = c.lse_out;
    p.lse_in = c.lse_in;
    p.S = S;
    p.slice_vecs = slice_vecs;
    p.stats = S ? (float *)((char *)c.ws + kPartialBytes) : nullptr;
    p.fix = S ? p.stats + 2 * (size_t)c.M * (size_t)S : nullptr;
    p.rowx = S ? p.fix + (size_t)c.M * (size_t)S : nullptr;
    p.ticket = nullptr;
    const int64_t fuse_max = tuning().fuse_max_bytes;
    if (reduction != CE_NONE && S == 0 &&
        (fuse_max < 0 || (int64_t)((size_t)c.M * (size_t)c.V * s) <= fuse_max))
        p.ticket = ticket_for(st);
    void *args[] = {&p};
    unsigned nunits = 0;
    if (S) {
        // split rows: slice statistics, then the per-row finish or the
        // epilogue over every slice, then (backward from lse) the target fix
        const cek::SplitKernels sk = split_kernels(c.dtype);
        const unsigned wgs = (unsigned)(c.M * S);
        if (c.op != cek::EPI_LSE_GRAD &&
            hipLaunchKernel(sk.stats, dim3(wgs), dim3(256), args, 0, st) != hipSuccess)
            return CE_ERR_HIP;
        const bool fwd = c.op == cek::EPI_NONE;
        if (hipLaunchKernel(fwd ? sk.finish : sk.epi[c.op], dim3(fwd ? (unsigned)c.M : wgs),
                            dim3(fwd ? 64 : 256), args, 0, st) != hipSuccess)
            return CE_ERR_HIP;
        if (c.op == cek::EPI_LSE_GRAD &&
            hipLaunchKernel(sk.fix, dim3((unsigned)((c.M + 3) / 4)), dim3(256), args, 0, st) !=
                hipSuccess)
            return CE_ERR_HIP;
        nunits = (unsigned)c.M;   // one partial per row
    } else {
        if (hipLaunchKernel(plan.k.fn, dim3((unsigned)plan.grid), dim3(plan.k.block), args, 0,
                            st) != hipSuccess)
            return CE_ERR_HIP;
        nunits = (unsigned)(plan.grid * plan.units_per_wg);
    }
    if (reduction != CE_NONE && !p.ticket) {
        // the fixed-order sum of the units' partials (same stream, after the grid)
        void *args2[] = {&p, &nunits};
        if (hipLaunchKernel(cek::sum_partials_fn(), dim3(1), dim3(64), args2, 0, st) != hipSuccess)
            return CE_ERR_HIP;
    }
    return CE_OK;
}

// ---- the library's own scratch (the entry point that allocates nothing) ----
// Room for what a forward's kernels keep beyond their inputs and outputs under
// the default plans: the fp64 partial sums of a mean or sum (at most
// kMaxPartials slots, the launch plan's cap) and the split-row statistics of
// up to kSplitMaxRows rows of kMaxSplit slices.  Nothing in it needs to start
// at zero: every slot a call reads was written earlier in the same call.
constexpr size_t kScratchBytes =
    kPartialBytes + (size_t)kSplitMaxRows * (kMaxSplit * kSplitBytesPerSlice + 4);
static_assert(kScratchBytes == CE_NOALLOC_SCRATCH_BYTES, "ce.h states the scratch size");
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

}  // namespace

// One copy per GPU, held until the process ends.  In host code `scratch` only
// names the symbol: kernels get the device address looked up below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
int scratch_address(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return CE_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return CE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CE_OK;
}

}  // namespace

namespace cek {
bool tuning_linear_library() { return tuning().linear_library; }
}  // namespace cek

extern "C" {

void ce_tuning_reload(void)
{
    tuning();   // the first read, if not done yet
    std::lock_guard<std::mutex> lk(g_tuning_mu);
    read_tuning(&g_tuning);
}

size_t ce_workspace_bytes(int64_t M, int64_t V, ce_dtype_t dtype, ce_reduction_t reduction)
{
    if (dtype != CE_F32 && dtype != CE_F16 && dtype != CE_BF16)
        return 0;
    if (reduction != CE_NONE && reduction != CE_MEAN && reduction != CE_SUM)
        return 0;
    if (M <= 0 || V < 1 || V > CE_MAX_V)
        return 0;
    // the worst-case window (a misaligned base) bounds the slices
    const int E = 16 / (int)elem_size(dtype);
    int sv = 0;
    const int S = split_slices(M, window_vectors(V, E, false), &sv);
    if (S > 0)
        return kPartialBytes + (size_t)M * (kMaxSplit * kSplitBytesPerSlice + 4);
    return reduction == CE_NONE ? 0 : kPartialBytes;
}

int ce_fwd(const void *logits, const int64_t *targets, int64_t M, int64_t V, ce_dtype_t dtype,
           ce_reduction_t reduction, float *out, void *workspace, size_t workspace_bytes,
           void *stream)
{
    Call c;
    c.logits = logits;
    c.targets = targets;
    c.M = M;
    c.V = V;
    c.dtype = (int)dtype;
    c.reduction = (int)reduction;
    c.out = out;
    c.ws = workspace;
    c.ws_bytes = workspace_bytes;
    return run(c, stream);
}

int ce_fwd_noalloc(const void *logits, const int64_t *targets, int64_t M, int64_t V,
                   ce_dtype_t dtype, ce_reduction_t reduction, float *out, void *stream)
{
    Call c;
    c.logits = logits;
    c.targets = targets;
    c.M = M;
    c.V = V;
    c.dtype = (int)dtype;
    c.reduction = (int)reduction;
    c.out = out;
    c.own_scratch = true;
    int rc = check_args(c);
    if (rc)
        return rc;
    size_t need = 0;
    planned_split(c, nullptr, &need);
    if (need > kScratchBytes)
        return CE_ERR_SCRATCH;
    if (need > 0) {
        rc = scratch_address(&c.ws);
        if (rc)
            return rc;
        c.ws_bytes = kScratchBytes;
    }
    return run(c, stream);
}

int ce_fwd_lse(const void *logits, const int64_t *targets, int64_t M, int64_t V,
               ce_dtype_t dtype, ce_reduction_t reduction, float *out, float *lse,
               void *workspace, size_t workspace_bytes, void *stream)
{
    if (M > 0 && !lse)
        return CE_ERR_NULL;
    Call c;
    c.logits = logits;
    c.targets = targets;
    c.M = M;
    c.V = V;
    c.dtype = (int)dtype;
    c.reduction = (int)reduction;
    c.out = out;
    c.lse_out = lse;
    c.ws = workspace;
    c.ws_bytes = workspace_bytes;
    return run(c, stream);
}

int ce_fwd_bwd_inplace(void *logits, const int64_t *targets, int64_t M, int64_t V,
                       ce_dtype_t dtype, ce_reduction_t reduction, float *loss_out,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    Call c;
    c.op = cek::EPI_GRAD;
    c.logits = logits;
    c.y = logits;
    c.targets = targets;
    c.M = M;
    c.V = V;
    c.dtype = (int)dtype;
    c.reduction = (int)reduction;
    c.out = loss_out;
    c.ws = workspace;
    c.ws_bytes = workspace_bytes;
    return run(c, stream);
}

int ce_bwd(const void *logits, const int64_t *targets, const float *lse, const float *dloss,
           int64_t M, int64_t V, ce_dtype_t dtype, ce_reduction_t reduction, void *grad,
           void *workspace, size_t workspace_bytes, void *stream)
{
    Call c;
    c.op = cek::EPI_LSE_GRAD;
    c.loss = false;
    c.logits = logits;
    c.targets = targets;
    c.lse_in = lse;
    c.dloss = dloss;
    c.M = M;
    c.V = V;
    c.dtype = (int)dtype;
    c.reduction = (int)reduction;
    c.y = grad;
    c.ws = workspace;
    c.ws_bytes = workspace ? workspace_bytes : 0;
    return run(c, stream);
}

int ce_softmax(const void *logits, int64_t M, int64_t V, ce_dtype_t dtype, int log_softmax,
               void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    Call c;
    c.op = log_softmax ? cek::EPI_LOGSOFTMAX : cek::EPI_SOFTMAX;
    c.loss = false;
    c.logits = logits;
    c.M = M;
    c.V = V;
    c.dtype = (int)dtype;
    c.y = out;
    c.lse_out = lse;
    c.ws = workspace;
    c.ws_bytes = workspace ? workspace_bytes : 0;
    return run(c, stream);
}

const char *ce_status_string(int status)
{
    switch (status) {
    case CE_OK: return "ok";
    case CE_ERR_NULL: return "a required pointer is NULL";
    case CE_ERR_SHAPE: return "bad shape (M < 0, V < 1, V too large, or size overflow)";
    case CE_ERR_DTYPE: return "unknown dtype";
    case CE_ERR_REDUCTION: return "unknown reduction";
    case CE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case CE_ERR_HIP: return "HIP runtime error or launch failure";
    case CE_ERR_ALIGNMENT:
        return "a pointer not aligned to its element size, or an output not at the logits' "
               "address modulo 16";
    case CE_ERR_ALIAS: return "an output overlaps another output or an input";
    case CE_ERR_SCRATCH:
        return "the call needs more scratch than the library's static per-device scratch "
               "holds (ce_fwd_noalloc)";
    default: return "unknown status";
    }
}

int ce_plan_describe(int64_t M, int64_t V, ce_dtype_t dtype, ce_reduction_t reduction, int op,
                     char *buf, size_t buf_len)
{
    if (!buf || !buf_len)
        return CE_ERR_NULL;
    if (dtype != CE_F32 && dtype != CE_F16 && dtype != CE_BF16)
        return CE_ERR_DTYPE;
    if (reduction != CE_NONE && reduction != CE_MEAN && reduction != CE_SUM)
        return CE_ERR_REDUCTION;
    if (M < 1 || V < 1 || V > CE_MAX_V)
        return CE_ERR_SHAPE;
    static const int ops[] = {cek::EPI_NONE, cek::EPI_GRAD, cek::EPI_SOFTMAX, cek::EPI_LOGSOFTMAX,
                              cek::EPI_LSE_GRAD};
    if (op < CE_OP_FWD || op > CE_OP_BWD)
        return CE_ERR_SHAPE;
    const int E = 16 / (int)elem_size(dtype);
    const bool aligned = V % E == 0;   // for a 16-byte aligned base
    int sv = 0;
    const int S = split_slices(M, window_vectors(V, E, aligned), &sv);
    if (S > 0) {
        std::snprintf(buf, buf_len, "split:%d slice=%d block=256 grid=%lld (with workspace)", S,
                      sv, (long long)M * S);
        return CE_OK;
    }
    Plan plan;
    int rc = make_plan(M, V, (int)dtype, ops[op], aligned, &plan);
    if (rc)
        return rc;
    static const char *names[] = {"rows", "wg", "stream", "wstream", "wg2"};
    std::snprintf(buf, buf_len, "%s:%d:%d%s%s%s block=%d grid=%lld occupancy=%d cus=%d",
                  names[plan.kind], plan.a, plan.b, plan.exact ? " exact" : "",
                  plan.nbuf == 2 ? " nbuf=2" : "", plan.blocked ? " blocked" : "", plan.k.block,
                  (long long)plan.grid, plan.occupancy, plan.cus);
    return CE_OK;
}

}  // extern "C"
