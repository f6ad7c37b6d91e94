// gemm.hip -- expert compute over the expert-grouped buffer: one projection,
// a grouped GEMM on the matrix cores.
//
// The MoonEP article (ncijnetwork.com), three-property list: views of the
// static buffer go straight to the computation, which finds each rank's rows
// grouped by expert (home experts, then the replicas the rank hosts).  Its
// explainer "memory" panel: a replica's weights sit in its prefetch slot, or,
// past the B slots, are read at the home expert.
//
//   y[r, n] = bf16( sum_k x[r, k] * W(r)[n, k] )
//
// with W(r) the [out_dim, in_dim] matrix at element w_offset of the weight row
// of r's segment.  A segment is a home expert (rows home_row_off[e] .. + keep[e]
// of rank e div L) or a replica (rows rep_row_off[j] .. + rep_count[j] of its
// host).  Segments are cut into tiles of BM rows that never cross a segment,
// so every tile multiplies by one weight matrix.
//
// Kernel: a persistent grid, one workgroup per CU.  Every workgroup first
// scans the per-segment tile counts into LDS (n_rep is known only on the
// device), then walks (tile, column-block) items.  Items are numbered in
// groups of kGroupM row tiles, the row tile running fastest inside a group,
// so any run of 32 consecutive items covers 8 row tiles and 4 column blocks
// (12 distinct operand slices per k-step instead of up to 29 when the column
// block runs fastest on a wide output).  The grid walks them in rounds of
// gridDim items, each XCD taking one run of consecutive items per round:
// the workgroups running together on one XCD share their A and B slices in
// that XCD's L2, and all XCDs stay within one window of the item space, so
// the weights they read at the same time are those of one or two segments
// and stay in the MALL.  Per item: BM x BN
// outputs; K advances BK at a time through a ring of S LDS stages filled by
// LDS-DMA (global_load_lds_dwordx4: no staging registers), with the 16-byte
// chunks of each row XOR-swizzled so that fragment reads are free of bank
// conflicts.  Each wave computes WM x WN outputs with (WM/32) x (WN/32)
// v_mfma_f32_32x32x16_bf16 accumulators (fp32); scheduling hints interleave
// the next k-step's fragment reads with the current MFMAs.  The tile is then
// rounded to bf16 (nearest even) and stored through LDS as 16-byte rows, one
// band of waves at a time.  The configuration used is at the end of the file.
//
// MFMA lane layouts (checked on gfx950): operand A lane l holds row l % 32,
// k = (l / 32) * 8 .. + 7; operand B lane l holds column l % 32, same k; the
// 32 x 32 fp32 result holds, in lane l and register r, row
// (r / 4) * 8 + (l / 32) * 4 + r % 4 and column l % 32.
#include "moonep_internal.hpp"

namespace moonep {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Row tiles per item group (the item order of the grouped GEMM).  Measured
// against 4 and against no grouping: best on the wide DeepSeek-V3-like
// projections, no change on the 2048-wide ones.
constexpr int kGroupM = 8;

template <int BM, int BN, int WM, int WN, int BK, int S>
struct GemmCfg {
    static constexpr int kBK = BK;                      // k per LDS stage (32 or 64)
    static constexpr int kStages = S;                   // LDS ring depth; S - 1 stages in flight
    static constexpr int kCpr = BK / 8;                 // 16-byte chunks per row
    static constexpr int kRpi = 64 / kCpr;              // rows per LDS-DMA load (1 KiB)
    static constexpr int kTM = WM / 32, kTN = WN / 32;  // 32 x 32 MFMA tiles per wave
    static constexpr int kWM = BM / WM, kWN = BN / WN;
    static constexpr int kWavesG = kWM * kWN;
    static constexpr int kThreads = kWavesG * 64;
    static constexpr int kRowBytes = BK * 2;
    static constexpr int kStageBytes = (BM + BN) * kRowBytes;
    static constexpr int kAInstr = BM / kRpi / kWavesG; // LDS-DMA loads per wave per stage
    static constexpr int kBInstr = BN / kRpi / kWavesG;
    static constexpr int kPerStage = kAInstr + kBInstr;
    static constexpr int kLdo = BN + 8;                 // epilogue LDS row, elements
    static constexpr int kOVec = WM * BN / 8 / kThreads;  // 16-byte stores per thread per band
    static_assert(BK == 32 || BK == 64, "stage depth");
    static_assert(S >= 2 && (S - 2) * kPerStage <= 63, "outstanding loads must fit vmcnt");
    static_assert(WM * kLdo * 2 <= S * kStageBytes, "an epilogue band must fit the ring");
    static_assert(kAInstr >= 1 && kBInstr >= 1 && kOVec >= 1, "tile too small for the block");
    static_assert(BM % (kRpi * kWavesG) == 0 && BN % (kRpi * kWavesG) == 0, "rows per DMA round");
    // chunk position of chunk c in row r: c ^ swz(r).  Rows of 128 bytes
    // (BK = 64) pair up in the 64 banks of 4 bytes, so swz takes row bits
    // 1..3: the fragment reads of 16 consecutive rows, which the LDS serves
    // together, land on 16 different 16-byte bank groups.  For 64-byte rows
    // (BK = 32) four rows share the banks and swz takes row bits 2..3.
    __device__ static constexpr int swz(int r) { return (r / (16 / kCpr)) % kCpr; }
};

// Exclusive scan of one int per thread over a block of NW waves.
template <int NW>
__device__ __forceinline__ int block_scan_excl(int v, int *tmp, int *total)
{
    const int lane = lane_id(), wid = (int)threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += o;
    }
    if (lane == 63)
        tmp[wid] = incl;
    __syncthreads();
    int base = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int t = tmp[w];
        base += w < wid ? t : 0;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return base + incl - v;
}

struct GemmArgs {
    const int32_t *plan;
    PlanLayout pl;
    const int32_t *wslot;
    int32_t R, E, L, C, nslots;
    int32_t in_dim, out_dim;
    const uint16_t *x, *w_home, *pool;
    int64_t w_stride, w_offset;
    uint16_t *y;
};

template <int BM, int BN, int WM, int WN, int BK, int S>
__global__ __launch_bounds__((GemmCfg<BM, BN, WM, WN, BK, S>::kThreads)) void expert_gemm_kernel(
    GemmArgs a)
{
    using G = GemmCfg<BM, BN, WM, WN, BK, S>;
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t *stage0 = lds;
    int32_t *seg_start = (int32_t *)((char *)lds + S * G::kStageBytes);  // [E + cap + 1]
    __shared__ int scan_tmp[G::kWavesG];

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int32_t cap = a.pl.cap;
    const int32_t nr_raw = a.plan[a.pl.header + MOONEP_PLAN_H_N_REP];
    const int32_t n_rep = nr_raw < 0 ? 0 : (nr_raw < cap ? nr_raw : cap);
    const int32_t nseg = a.E + n_rep;

    // ---- segment tile counts, scanned into seg_start ----------------------
    // segment s < E: home expert s; s >= E: replica s - E.  A bad table entry
    // makes an empty segment, so every access below stays in bounds.
    auto seg_len = [&](int32_t s) -> int32_t {
        if (s < a.E) {
            const int32_t off = a.plan[a.pl.home_row_off + s], n = a.plan[a.pl.keep + s];
            return (off >= 0 && n >= 0 && off <= a.C - n) ? n : 0;
        }
        const int32_t j = s - a.E;
        const int32_t h = a.plan[a.pl.rep_host + j], e = a.plan[a.pl.rep_expert + j];
        const int32_t off = a.plan[a.pl.rep_row_off + j], n = a.plan[a.pl.rep_count + j];
        return (h >= 0 && h < a.R && e >= 0 && e < a.E && off >= 0 && n >= 0 && off <= a.C - n)
                   ? n : 0;
    };
    const int32_t per = (nseg + G::kThreads - 1) / G::kThreads;
    const int32_t s0 = tid * per;
    int32_t mine = 0;
    for (int32_t s = s0; s < s0 + per && s < nseg; ++s) {
        const int32_t len = seg_len(s);
        mine += len > 0 ? (len + BM - 1) / BM : 0;
    }
    int32_t total_tiles = 0;
    int32_t run = block_scan_excl<G::kWavesG>(mine, scan_tmp, &total_tiles);
    for (int32_t s = s0; s < s0 + per && s < nseg; ++s) {
        seg_start[s] = run;
        const int32_t len = seg_len(s);
        run += len > 0 ? (len + BM - 1) / BM : 0;
    }
    if (tid == 0)
        seg_start[nseg] = total_tiles;
    __syncthreads();

    // ---- items of this workgroup's XCD -------------------------------------
    const int32_t nbn = (a.out_dim + BN - 1) / BN;  // the last block may be part-empty
    const int64_t items = (int64_t)total_tiles * nbn;
    // workgroup b runs on XCD b % 8; the XCD-x workgroups take the slots
    // after those of XCDs 0..x-1 in each round (XCD x holds ceil((P - x)/8))
    const int xcd = (int)(blockIdx.x % 8), q = (int)(blockIdx.x / 8);
    const int P = (int)gridDim.x;
    int slot = q;
    for (int x = 0; x < xcd; ++x)
        slot += (P - x + 7) / 8;
    const int32_t nk = a.in_dim / G::kBK;
    const int wm = wave / G::kWN, wn = wave % G::kWN;
    int log_nseg = 0;
    while ((1 << log_nseg) < nseg + 1)
        ++log_nseg;

    for (int64_t it = slot; it < items; it += P) {
        // item -> (row tile t, column block nb): group gi holds row tiles
        // [gi*kGroupM, gi*kGroupM + gm), gm < kGroupM only for the last group
        const int64_t gi = it / ((int64_t)kGroupM * nbn);
        const int32_t within = (int32_t)(it - gi * ((int64_t)kGroupM * nbn));
        const int32_t gleft = total_tiles - (int32_t)gi * kGroupM;
        const int32_t gm = gleft < kGroupM ? gleft : kGroupM;
        const int32_t t = (int32_t)gi * kGroupM + within % gm;
        const int32_t nb = within / gm;
        // segment holding tile t: last s with seg_start[s] <= t (fixed-depth search)
        int32_t s = 0;
        for (int b = log_nseg - 1; b >= 0; --b) {
            const int32_t c = s + (1 << b);
            if (c < nseg && seg_start[c] <= t)
                s = c;
        }
        const int32_t mt = t - seg_start[s];
        int64_t row0;
        int32_t len;
        const uint16_t *wbase;
        if (s < a.E) {
            row0 = (int64_t)(s / a.L) * a.C + a.plan[a.pl.home_row_off + s];
            len = seg_len(s);
            wbase = a.w_home + (int64_t)s * a.w_stride;
        } else {
            const int32_t j = s - a.E;
            row0 = (int64_t)a.plan[a.pl.rep_host + j] * a.C + a.plan[a.pl.rep_row_off + j];
            len = seg_len(s);
            const int32_t ws = a.wslot[j];
            wbase = (ws >= 0 && ws < a.nslots)
                        ? a.pool + (int64_t)ws * a.w_stride
                        : a.w_home + (int64_t)a.plan[a.pl.rep_expert + j] * a.w_stride;
        }
        wbase += a.w_offset;
        const int64_t m0 = row0 + (int64_t)mt * BM;
        const int32_t mrows = len - mt * BM < BM ? len - mt * BM : BM;
        const int64_t n0 = (int64_t)nb * BN;

        // LDS layout of a stage: A rows then B rows, BK bf16 (2 BK bytes) each,
        // 16-byte chunk c of row r stored at chunk position c ^ swz(r).  One
        // LDS-DMA load per wave fills kRpi rows (1 KiB, lane i -> byte 16 i):
        // lane i brings chunk (i % kCpr) ^ swz(r) of row r = kRpi g + i / kCpr.
        const int dma_row = lane / G::kCpr, dma_pos = lane % G::kCpr;
        uint32_t a_off[G::kAInstr], b_off[G::kBInstr];
#pragma unroll
        for (int v = 0; v < G::kAInstr; ++v) {
            const int row = (v * G::kWavesG + wave) * G::kRpi + dma_row;
            const int chunk = dma_pos ^ G::swz(row);
            a_off[v] = (uint32_t)((row < mrows ? row : 0) * a.in_dim * 2 + chunk * 16);
        }
#pragma unroll
        for (int v = 0; v < G::kBInstr; ++v) {
            const int row = (v * G::kWavesG + wave) * G::kRpi + dma_row;
            const int chunk = dma_pos ^ G::swz(row);
            b_off[v] = (uint32_t)((n0 + row < a.out_dim ? row : 0) * a.in_dim * 2 + chunk * 16);
        }
        const char *a_base = (const char *)(a.x + m0 * a.in_dim);
        const char *b_base = (const char *)(wbase + n0 * a.in_dim);
        char *lds_b = (char *)stage0;
        auto issue = [&](int32_t kt, int st) {
            char *dst = lds_b + st * G::kStageBytes + wave * 1024;
            const char *ap = a_base + (int64_t)kt * G::kRowBytes;
            const char *bp = b_base + (int64_t)kt * G::kRowBytes;
#pragma unroll
            for (int v = 0; v < G::kAInstr; ++v)
                __builtin_amdgcn_global_load_lds(
                    (const void *)(ap + a_off[v]),
                    (__attribute__((address_space(3))) void *)(dst + v * G::kWavesG * 1024), 16, 0, 0);
#pragma unroll
            for (int v = 0; v < G::kBInstr; ++v)
                __builtin_amdgcn_global_load_lds(
                    (const void *)(bp + b_off[v]),
                    (__attribute__((address_space(3))) void *)(dst + BM * G::kRowBytes +
                                                               v * G::kWavesG * 1024),
                    16, 0, 0);
        };
        // fragment of 32 rows from row0 (a multiple of 32) at k-step ks: lane l
        // reads row row0 + l % 32, chunk 2 ks + l / 32
        const int fr = lane & 31, fsw = G::swz(lane & 31), fhalf = lane >> 5;
        auto frag = [&](const char *base, int row0, int ks) -> bf16x8 {
            return *(const bf16x8 *)(base + (row0 + fr) * G::kRowBytes +
                                     (((2 * ks + fhalf) ^ fsw) << 4));
        };

        f32x16 acc[G::kTM][G::kTN];
#pragma unroll
        for (int i = 0; i < G::kTM; ++i)
#pragma unroll
            for (int j = 0; j < G::kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;

        // ring of S stages, S - 1 in flight: stage kt lives in slot kt % S
#pragma unroll
        for (int st = 0; st + 1 < S; ++st)
            if (st < nk)
                issue(st, st);
        for (int32_t kt = 0; kt < nk; ++kt) {
            // this wave's loads of stage kt have landed once at most the later
            // stages' loads are outstanding
            if (kt + S - 2 < nk) {
                if constexpr (S == 2)
                    __builtin_amdgcn_s_waitcnt(0x0F70);
                else if constexpr (S == 3)
                    __builtin_amdgcn_s_waitcnt(0x0F70 | (G::kPerStage & 15) |
                                               ((G::kPerStage >> 4) << 14));
                else
                    __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * G::kPerStage) & 15) |
                                               (((2 * G::kPerStage) >> 4) << 14));
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);
            }
            __syncthreads();  // every wave's part of stage kt is visible; slot (kt-1) % S is free
            if (kt + S - 1 < nk)
                issue(kt + S - 1, (kt + S - 1) % S);
            const char *sa = lds_b + (kt % S) * G::kStageBytes;
            const char *sb = sa + BM * G::kRowBytes;
            bf16x8 fa[2][G::kTM], fb[2][G::kTN];
#pragma unroll
            for (int i = 0; i < G::kTM; ++i)
                fa[0][i] = frag(sa, wm * WM + i * 32, 0);
#pragma unroll
            for (int j = 0; j < G::kTN; ++j)
                fb[0][j] = frag(sb, wn * WN + j * 32, 0);
#pragma unroll
            for (int ks = 0; ks < G::kBK / 16; ++ks) {
                const int cur = ks & 1, nxt = cur ^ 1;
                if (ks + 1 < G::kBK / 16) {
#pragma unroll
                    for (int i = 0; i < G::kTM; ++i)
                        fa[nxt][i] = frag(sa, wm * WM + i * 32, ks + 1);
#pragma unroll
                    for (int j = 0; j < G::kTN; ++j)
                        fb[nxt][j] = frag(sb, wn * WN + j * 32, ks + 1);
                }
#pragma unroll
                for (int i = 0; i < G::kTM; ++i)
#pragma unroll
                    for (int j = 0; j < G::kTN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j],
                                                                            acc[i][j], 0, 0, 0);
            }
            // Schedule: the first k-step's fragments, then each later k-step's
            // fragment reads spread between the MFMAs of the step before, so LDS
            // latency hides under the matrix work.
            constexpr int kFr = G::kTM + G::kTN, kMf = G::kTM * G::kTN;
            __builtin_amdgcn_sched_group_barrier(0x100, kFr, 0);
#pragma unroll
            for (int ks = 0; ks + 1 < G::kBK / 16; ++ks) {
#pragma unroll
                for (int r = 0; r < kFr; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, kMf / kFr, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
        }
        __syncthreads();  // every wave is done with the ring before the epilogue reuses it

        // ---- epilogue: one band of wave rows at a time through LDS ------------
        uint16_t *so = stage0;
#pragma unroll
        for (int band = 0; band < G::kWM; ++band) {
            if (wm == band) {
#pragma unroll
                for (int i = 0; i < G::kTM; ++i)
#pragma unroll
                    for (int j = 0; j < G::kTN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; r += 2) {
                            const int row = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                            const int col = wn * WN + j * 32 + (lane & 31);
                            const uint32_t p = pack_bf16(acc[i][j][r], acc[i][j][r + 1]);
                            so[row * G::kLdo + col] = (uint16_t)(p & 0xFFFFu);
                            so[(row + 1) * G::kLdo + col] = (uint16_t)(p >> 16);
                        }
            }
            __syncthreads();
#pragma unroll
            for (int v = 0; v < G::kOVec; ++v) {
                const int idx = tid + v * G::kThreads;
                const int row = idx / (BN / 8), c = idx % (BN / 8);
                const int grow = band * WM + row;
                if (grow < mrows && n0 + c * 8 < a.out_dim)
                    *(u32x4 *)(a.y + (m0 + grow) * a.out_dim + n0 + c * 8) =
                        *(const u32x4 *)(so + row * G::kLdo + c * 8);
            }
            __syncthreads();
        }
    }
}

namespace {

template <int BM, int BN, int WM, int WN, int BK, int S>
int run_gemm(const GemmArgs &ga, hipStream_t st)
{
    using G = GemmCfg<BM, BN, WM, WN, BK, S>;
    const size_t lds = (size_t)S * G::kStageBytes + (size_t)(ga.E + ga.pl.cap + 1) * 4;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MOONEP_ERR_HIP;
    // Raise the kernel's dynamic-LDS limit once per device, to what the largest
    // allowed E and R need, so later calls with other shapes fit as well.
    static bool raised[64] = {};
    if (dev < 0 || dev >= 64 || !raised[dev]) {
        const size_t most = (size_t)S * G::kStageBytes + (size_t)(2 * kMaxExperts + kMaxRanks + 1) * 4;
        if (hipFuncSetAttribute((const void *)expert_gemm_kernel<BM, BN, WM, WN, BK, S>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)most) != hipSuccess)
            return MOONEP_ERR_HIP;
        if (dev >= 0 && dev < 64)
            raised[dev] = true;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (expert_gemm_kernel<BM, BN, WM, WN, BK, S>),
                                                     G::kThreads, lds) != hipSuccess)
        return MOONEP_ERR_HIP;
    const int grid = cus * (per_cu > 0 ? per_cu : 1);
    hipLaunchKernelGGL((expert_gemm_kernel<BM, BN, WM, WN, BK, S>), dim3(grid), dim3(G::kThreads), lds, st, ga);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace

constexpr int kGemmBM = 256, kGemmBN = 256, kGemmWM = 128, kGemmWN = 64, kGemmBK = 64,
              kGemmStages = 2;

int gemm_out_align() { return 128; }

int launch_expert_gemm(const moonep_shape &s, const int32_t *plan, const int32_t *wslot, int32_t B,
                       int32_t in_dim, int32_t out_dim, const uint16_t *x, const uint16_t *w_home,
                       const uint16_t *pool, int64_t w_stride, int64_t w_offset, uint16_t *y,
                       hipStream_t st)
{
    if ((int64_t)s.R * s.S * s.K == 0)
        return MOONEP_OK;
    GemmArgs ga;
    ga.plan = plan;
    ga.pl = plan_layout(s.E, s.R);
    ga.wslot = wslot;
    ga.R = s.R;
    ga.E = s.E;
    ga.L = s.E / s.R;
    ga.C = s.S * s.K;
    ga.nslots = s.R * B;
    ga.in_dim = in_dim;
    ga.out_dim = out_dim;
    ga.x = x;
    ga.w_home = w_home;
    ga.pool = pool;
    ga.w_stride = w_stride;
    ga.w_offset = w_offset;
    ga.y = y;
    return run_gemm<kGemmBM, kGemmBN, kGemmWM, kGemmWN, kGemmBK, kGemmStages>(ga, st);
}

}  // namespace moonep
