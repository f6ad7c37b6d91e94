// moonep_internal.hpp -- layouts and gfx950 device helpers shared by the
// kernels of libmoonep.  Nothing here is part of the public C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moonep.h"

namespace moonep {

// ---------------------------------------------------------------------------
// Limits and launch geometry
// ---------------------------------------------------------------------------

constexpr int kMaxExperts = 1024;  // on-chip plan tables
constexpr int kMaxRanks = 512;
constexpr int kBlock = 256;        // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
// Wave segments (one wave each) for route_stats and the plan: NK / 512 of
// them, kept between 1024 and 2048.  route_stats + plan measured best so on
// gfx950: 1024 segments of 256 entries on a 262K-entry routing (27.4 us,
// against 28.2 at 2048 and 30-31 at 512), 2048 of 512 entries on 1M-entry
// ones (57.5 us against 60.7 at 1024 and 65.6 at 4096 on the 256-expert
// shape; 42.0 against 46.4 and 45.9 on the 128-expert one).
constexpr int kMinSegments = 1024, kMaxSegments = 2048, kSegmentEntries = 512;
constexpr int kChunkBatch = 16;        // 64-entry chunks loaded ahead per wave
constexpr size_t kCtlBytes = 256;      // workspace control block

// Workspace control block (int32 words): the sticky device error word.
enum { kCtlError = 0 };

struct WsLayout {
    int64_t nk;      // routed entries R*S*K
    int32_t segw;    // entries per wave segment (multiple of 64)
    int32_t nseg;    // wave segments
    size_t hist_off; // byte offset of the [E][nseg] int32 counts / bases
    size_t bytes;    // total workspace bytes
};

inline WsLayout ws_layout(const moonep_shape &s)
{
    WsLayout w{};
    w.nk = (int64_t)s.R * s.S * s.K;
    int64_t target = w.nk / kSegmentEntries;
    target = target < kMinSegments ? kMinSegments : (target > kMaxSegments ? kMaxSegments : target);
    int64_t per = (w.nk + target - 1) / target;
    per = ((per + 63) / 64) * 64;
    if (per < 64)
        per = 64;
    w.segw = (int32_t)per;
    w.nseg = (int32_t)((w.nk + per - 1) / per);
    w.hist_off = kCtlBytes;
    size_t hist = (size_t)s.E * (size_t)w.nseg * 4;
    w.bytes = kCtlBytes + ((hist + 255) / 256) * 256;
    return w;
}

struct PlanLayout {
    int32_t words, cap;
    int32_t header, rep_expert, rep_host, rep_count, rep_spill_off, rep_row_off;
    int32_t spill, keep, home_row_off, rep_first, rep_cnt, exp_rep_list;
    int32_t load, rank_rep_first, rank_rep_cnt;
};

__host__ __device__ inline PlanLayout plan_layout(int32_t E, int32_t R)
{
    PlanLayout p{};
    p.cap = E + R;
    int32_t o = 0;
    p.header = o; o += 16;
    p.rep_expert = o; o += p.cap;
    p.rep_host = o; o += p.cap;
    p.rep_count = o; o += p.cap;
    p.rep_spill_off = o; o += p.cap;
    p.rep_row_off = o; o += p.cap;
    p.spill = o; o += E;
    p.keep = o; o += E;
    p.home_row_off = o; o += E;
    p.rep_first = o; o += E;
    p.rep_cnt = o; o += E;
    p.exp_rep_list = o; o += E;
    p.load = o; o += R;
    p.rank_rep_first = o; o += R;
    p.rank_rep_cnt = o; o += R;
    p.words = o;
    return p;
}

// Bits needed to tell expert ids 0..E-1 apart.
__host__ __device__ inline int expert_bits(int32_t E)
{
    int b = 0;
    while ((1 << b) < E)
        ++b;
    return b;
}

// ---------------------------------------------------------------------------
// Device helpers (wave64)
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// popcount of the bits of m below this lane.
__device__ __forceinline__ int count_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Orders LDS traffic between the lanes of one wave (no hardware barrier).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// For G chunks of keys at once: narrows same[u], which enters as the mask of
// lanes that take part in chunk u, to those whose key equals this lane's.
// One ballot per key bit, so the cost does not depend on how the keys
// repeat; the G chunks' chains run side by side.
template <int G>
__device__ __forceinline__ void match_lanes(const int32_t (&key)[G], int nbits, uint64_t (&same)[G])
{
    for (int b = 0; b < nbits; ++b) {
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const bool on = (key[u] >> b) & 1;
            const uint64_t set = ballot(on);
            same[u] &= on ? set : ~set;
        }
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    f2 v = {lo, hi};
    b2 r = __builtin_convertvector(v, b2);
    return __builtin_bit_cast(uint32_t, r);
}

// bf16 bits of the exact product a*b (a fp32, b bf16-valued fp32), rounded
// once to nearest even.  The fp32 product p is off by err = fma(a,b,-p)
// exactly; only when p sits on a bf16 halfway point does err decide.
__device__ __forceinline__ uint32_t bf16_of_exact_product(float a, float b)
{
    const float p = a * b;
    const float err = __builtin_fmaf(a, b, -p);
    const uint32_t u = __float_as_uint(p);
    if ((u & 0xFFFFu) == 0x8000u && err != 0.0f) {
        const bool away = (err > 0.0f) == (p > 0.0f);
        return (u >> 16) + (away ? 1u : 0u);
    }
    const uint32_t w = pack_bf16(p, 0.0f);
    return w & 0xFFFFu;
}

// bf16 bits of a double, rounded once to nearest even: round to fp32 with
// round-to-odd (truncate toward zero, then set the last bit if anything was
// dropped), then to bf16 with round-to-nearest-even.  Rounding to odd at 24
// bits, at least two bits more than bf16's 8, makes the second rounding land
// where a direct rounding of the double would (Boldo and Melquiond, "Emulation
// of FMA and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE Trans. Computers 2008).
__device__ __forceinline__ uint32_t bf16_of_double(double d)
{
    float f = (float)d;
    if ((double)f != d && d == d) {
        uint32_t u = __float_as_uint(f);
        if (__builtin_fabs((double)f) > __builtin_fabs(d))
            u -= 1;  // one fp32 step toward zero
        u |= 1u;
        f = __uint_as_float(u);
    }
    return pack_bf16(f, 0.0f) & 0xFFFFu;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// Cross-lane steps on DPP (data-parallel primitives of the VALU): each is one
// vector instruction with no LDS round trip.  row_shr:n reads lane i - n of
// the same 16-lane row (zero when that lane is outside the row);
// row_bcast:15 and row_bcast:31 (gfx9) hand the last lane of row r - 1, or
// lane 31, to the rows the row mask enables.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118,
              kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive sum over lanes 0..l of v, in lane l (every lane of the wave active).
__device__ __forceinline__ int32_t wave_incl_sum(int32_t v)
{
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false);  // rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false);  // rows 2 and 3
    return v;
}

// Largest v over the wave, for v >= 0 (every lane active).
__device__ __forceinline__ int32_t wave_max_nonneg(int32_t v)
{
    v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// Exclusive scan over a block of kBlock threads of one int per thread.
// `tmp` must hold kWaves ints of LDS.  Returns the exclusive prefix; *total
// receives the block total.
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp, int *total)
{
    const int lane = lane_id();
    const int wid = (int)threadIdx.x >> 6;
    const int incl = wave_incl_sum(v);
    if (lane == 63)
        tmp[wid] = incl;
    __syncthreads();
    int base = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int t = tmp[w];
        if (w < wid)
            base += t;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return base + incl - v;
}

}  // namespace moonep
