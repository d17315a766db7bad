// Launch schedules of the factorization and quantize stages: which
// workgroup of a launch does what.  Plain integer arithmetic shared by the
// kernels (device), the launchers (host) and a host-only test build, so the
// checks on the CPU run this very code.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define GPTQ_HD __host__ __device__
#else
#define GPTQ_HD
#endif

namespace gptq {
namespace sched {

template <typename T>
GPTQ_HD inline T min_of(T a, T b) { return a < b ? a : b; }
template <typename T>
GPTQ_HD inline T max_of(T a, T b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// Factorization: blocked reverse Cholesky of G (T tiles of 64 per side) with
// the inverse carried along, one launch per step k.  The launch of step k
// holds, by workgroup index b:
//   b <  nchain          the diagonal block and panel of step k+1: workgroup
//                        b factors the diagonal block itself and forms panel
//                        tile t = b;
//   b == nchain          copies M_kk into G_kk;
//   b >  nchain          rest item b - nchain - 1: one tile of step k's
//                        update (rest_tile).
// Steps are paired from kPairMinTiles tiles on: an even launch defers its
// update of the rest, the next launch applies both steps as one 128-deep
// product per tile.
// ---------------------------------------------------------------------------
constexpr int kPairMinTiles = 128;

struct CholLaunch {
    int nchain;      // diagonal-block + panel workgroups (0 in the last launch)
    int64_t n_rest;  // rest items
    int64_t grid;    // workgroups of the launch
};

GPTQ_HD inline bool chol_paired(int T) { return T >= kPairMinTiles; }

// Lower tiles below row k except column and row block k+1 (those are
// updated by the diagonal-block workgroups of the same launch, in
// registers).
GPTQ_HD inline int64_t rest_tiles(int k, int T) {
    const int64_t all = (int64_t)T * (T + 1) / 2 - (int64_t)(k + 1) * (k + 2) / 2;
    return (k + 1 < T) ? all - T : all;
}

// Rest item b of step k, row-major over rows i >= k+2 with j in 0..i
// without k+1: returns the tile (i, j).
GPTQ_HD inline void rest_tile(int k, int64_t b, int64_t& i, int64_t& j) {
    // rows before row r contribute r(r-1)/2 - (k+1)(k+2)/2 items; start from
    // the integer square root of 8(b + c0) + 1 and correct exactly
    const int64_t c0 = (int64_t)(k + 1) * (k + 2) / 2;
    const int64_t v = 8 * (b + c0) + 1;
    int64_t lo = 0, hi = 1;
    while (hi * hi <= v) hi <<= 1;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if (mid * mid <= v) lo = mid;
        else hi = mid;
    }
    int64_t r = (1 + lo) / 2;
    while (r * (r - 1) / 2 - c0 > b) --r;
    while ((r + 1) * r / 2 - c0 <= b) ++r;
    i = r;
    const int64_t jj = b - (r * (r - 1) / 2 - c0);
    j = (jj < k + 1) ? jj : jj + 1;
}

GPTQ_HD inline CholLaunch chol_launch(int k, int T, bool paired) {
    CholLaunch g;
    g.nchain = (k + 1 < T) ? max_of(T - 1, 1) : 0;
    g.n_rest = (paired && (k % 2 == 0)) ? 0 : rest_tiles(k, T);
    g.grid = g.nchain + 1 + g.n_rest;
    return g;
}

// ---------------------------------------------------------------------------
// Quantize stage: the launch of lazy block [b0, b1) sweeps the block on
// n_sweep workgroups and applies the previous block's update to the columns
// [c_begin, d_in) in units of kFarRows rows x kFarStrip columns (unit u:
// row tile u / nstrip, strip u % nstrip).  The units are dealt out as
// contiguous ranges: each sweeping workgroup takes per_sweep units after its
// sweep (which takes about `sweep_units` units' time: at 4096 x 4096 a
// sweep of 64 rows by 128 columns lasts about 24 us, a unit of the split
// update about 3.9 us when every CU updates, kSweepUnits; one of the fp32
// update about 5 us, kSweepUnitsF32), the far-only workgroups share the rest
// evenly; a range is walked in sub-tiles of at most kFarCols columns that
// stay inside one row tile.
// ---------------------------------------------------------------------------
constexpr int kFarRows = 128;
constexpr int kFarCols = 256;
constexpr int kFarStrip = 64;
constexpr double kSweepUnits = 6.0;
constexpr double kSweepUnitsF32 = 3.0;

struct FarSplit {
    int64_t c_begin;
    int64_t n_units;
    int nstrip;     // strips per row tile
    int per_sweep;  // units of each sweeping workgroup
    int q, r;       // far-only workgroups: q units each, the first r one more
};

// Fills the split of n_units over n_sweep sweeping workgroups and the other
// CUs (one workgroup per CU); returns the number of far-only workgroups.
GPTQ_HD inline int far_split(int64_t n_units, int n_sweep, int n_cu, FarSplit& fs,
                             double sweep_units = kSweepUnits) {
    fs.n_units = n_units;
    fs.per_sweep = 0;
    fs.q = fs.r = 0;
    if (n_units <= 0) return 0;
    const int n_far = max_of(0, n_cu - n_sweep);
    if (n_far == 0) {  // more sweeping workgroups than CUs: they do it all
        fs.per_sweep = (int)((n_units + n_sweep - 1) / n_sweep);
        return 0;
    }
    const double t = ((double)n_units + n_sweep * sweep_units) / (double)(n_sweep + n_far);
    const double ps = t - sweep_units;
    fs.per_sweep = ps > 0.0 ? (int)ps : 0;  // floor of a non-negative value
    const int64_t rest = n_units - (int64_t)n_sweep * fs.per_sweep;
    const int nf = (int)min_of<int64_t>(n_far, rest);
    if (nf > 0) {
        fs.q = (int)(rest / nf);
        fs.r = (int)(rest % nf);
    }
    return nf;
}

// Units [u0, u1) of workgroup b (b < n_sweep: a sweeping workgroup).
GPTQ_HD inline void far_units(const FarSplit& fs, int b, int n_sweep, int64_t& u0, int64_t& u1) {
    if (b < n_sweep) {
        u0 = min_of<int64_t>((int64_t)b * fs.per_sweep, fs.n_units);
        u1 = min_of<int64_t>(u0 + fs.per_sweep, fs.n_units);
    } else {
        const int f = b - n_sweep;
        u0 = (int64_t)n_sweep * fs.per_sweep + (int64_t)f * fs.q + min_of(f, fs.r);
        u1 = u0 + fs.q + (f < fs.r ? 1 : 0);
    }
}

// The sub-tile that starts at unit u of a range ending at u1: row tile rt,
// columns [c0, c_end), and the units it covers (ns).
struct FarSub {
    int64_t rt;
    int64_t c0, c_end;
    int ns;
};

GPTQ_HD inline FarSub far_sub(const FarSplit& fs, int64_t u, int64_t u1, int64_t d_in) {
    FarSub t;
    t.rt = u / fs.nstrip;
    const int st = (int)(u - t.rt * fs.nstrip);
    t.ns = (int)min_of<int64_t>(min_of(kFarCols / kFarStrip, fs.nstrip - st), u1 - u);
    t.c0 = fs.c_begin + (int64_t)st * kFarStrip;
    t.c_end = min_of<int64_t>(d_in, t.c0 + (int64_t)t.ns * kFarStrip);
    return t;
}

}  // namespace sched
}  // namespace gptq
