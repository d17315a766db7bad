// Stage 1: H += 2 X X^T on the lower triangle (aicassindra.com
// "tm_gptq_math", "Why it is second-order: the Hessian").
//
// One workgroup per lower-triangle tile (I >= J) of H: 128x128 on four
// waves for narrow layers; for wide ones 256x256 on sixteen waves, or
// 192x192 on twelve (nine compute waves, three loader waves) where 256-wide
// tiles would leave CUs idle.  Every computing wave keeps one 64x64 quarter
// as 2x2 MFMA 32x32 accumulators.  Token slabs of X rows I
// and J are staged through LDS; products run on MFMA with fp32 accumulation
// (f16 inputs: 32x32x16 f16, exact products; f32 inputs: 32x32x2 f32).  Each
// launch adds its token range (one chunk, or up to kMaxChunks chunks held in
// separate buffers) into H once at the end.
// The MFMA instruction sequence over the tokens is the same for every tile,
// slab size and prefetch depth (zero-padded tails add exact zeros), so the
// sums are the same bits whichever kernel a shape takes.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ void tile_of(int b, int& I, int& J) {
    int i = (int)((sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
    while ((i + 1) * (i + 2) / 2 <= b) ++i;
    while (i * (i + 1) / 2 > b) --i;
    I = i;
    J = b - i * (i + 1) / 2;
}

// Adds 2*acc into the lower triangle of H for one wave's 64x64 quarter.  The
// old values of a 32-row half are all loaded before any of them is stored,
// so a wave waits for memory twice rather than once per element.  Entries
// past n or above the diagonal load from a clamped, always valid address
// (measured faster than skipping their loads) and are not stored.  Addresses
// are a wave-uniform row base plus an unsigned 32-bit offset (at most
// 64 n < 2^31 for any width whose H fits in memory).
template <bool kSet>
__device__ __forceinline__ void store_quarter(float* __restrict__ H, int64_t n, int r0, int c0,
                                              const float16v (&acc)[2][2], int lane) {
    const int ni = (int)n;
    const int rb = min(r0, ni - 1);
    float* __restrict__ base = H + (int64_t)rb * n;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float old[2][16] = {};
        if (!kSet) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = r0 + 32 * m + acc32_row(v, lane);
                    const int col = c0 + 32 * q + (lane & 31);
                    const int rr = min(row, ni - 1), cc = min(col, rr);
                    old[q][v] = base[(unsigned)((rr - rb) * ni + cc)];
                }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = r0 + 32 * m + acc32_row(v, lane);
                const int col = c0 + 32 * q + (lane & 31);
                if (row < ni && col <= row)
                    base[(unsigned)((row - rb) * ni + col)] = kSet ? 2.0f * acc[m][q][v] : old[q][v] + 2.0f * acc[m][q][v];
            }
    }
}

// ---------------------------------------------------------------------------
// float16 inputs
//
// Each thread keeps kDepth slabs of kK tokens in flight in registers
// (static register sets, the slab loop unrolled by kDepth) while the MFMAs
// consume the current slab from one of two LDS buffers.  The loads of a full
// slab are unconditional and every tile issues the same ones, so that before
// each LDS stash the compiler waits only for the oldest set in flight (with
// per-piece bounds branches it drained every load and the prefetch bought
// nothing).  Tiles are dealt out so that each XCD (workgroups are
// dispatched round-robin over the 8 XCDs) takes a contiguous run of a
// super-tile order of the lower triangle, keeping the X panels it reads
// few and resident in its own L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kSuper = 4;  // super-tile edge, in tiles

// The token chunks of one call: chunk c holds the call's tokens
// [c * spc * slab, (c + 1) * spc * slab) at p[c] (every chunk the same row
// stride), so that one launch sums several chunks before its single add into
// H.  spc = 0: one chunk, at X.
constexpr int kMaxChunks = 32;
struct XChunks {
    const half_t* p[kMaxChunks];
};

// Tile t of the super-tile order: super-rows P (kSuper tile rows each), in
// each super-row the super-tiles Q <= P left to right, in each super-tile the
// tiles row by row (only J <= I on the diagonal super-tile).
__host__ __device__ inline void tile_of_super(int t, int T, int& I, int& J) {
    const int SP = (T + kSuper - 1) / kSuper;
    for (int P = 0; P < SP; ++P) {
        const int r0 = P * kSuper, r1 = min(T, r0 + kSuper);
        for (int Q = 0; Q <= P; ++Q) {
            const int c0 = Q * kSuper, c1 = min(T, c0 + kSuper);
            int cnt = 0;
            if (Q < P) {
                cnt = (r1 - r0) * (c1 - c0);
                if (t < cnt) {
                    I = r0 + t / (c1 - c0);
                    J = c0 + t % (c1 - c0);
                    return;
                }
            } else {
                const int m = r1 - r0;
                cnt = m * (m + 1) / 2;
                if (t < cnt) {
                    int i = 0;
                    while ((i + 1) * (i + 2) / 2 <= t) ++i;
                    I = r0 + i;
                    J = c0 + (t - i * (i + 1) / 2);
                    return;
                }
            }
            t -= cnt;
        }
    }
    I = J = 0;  // not reached for t < T(T+1)/2
}

// Thread tid of kThr moves the half8 pieces of a kTl x kK slab: piece i is
// row tid / (kK/8) + i * (kThr / (kK/8)), halves (tid % (kK/8)) * 8 .. +8.
template <int kTl, int kThr, int kK>
struct Slab {
    static constexpr int kChunks = kK / 8;              // half8 pieces per row
    static constexpr int kRowsPerPass = kThr / kChunks;
    static constexpr int kPieces = kTl / kRowsPerPass;  // per thread
    static constexpr int kLd = kK + 8;                  // padded LDS row (halves)
};
template <int kTl, int kThr, int kK>
using SlabRegs = half8[Slab<kTl, kThr, kK>::kPieces];

// A slab whose tokens all lie below ntok, with 16-byte aligned rows: one
// unconditional 16-byte load per piece.  Rows past n are clamped to row n-1:
// they only feed accumulator entries that are never stored.
template <int kTl, int kThr, int kK>
__device__ __forceinline__ void fetch_full(SlabRegs<kTl, kThr, kK>& v, const half_t* __restrict__ X, int64_t n,
                                           int64_t ldx, int r0, int64_t k0, int tid) {
    using S = Slab<kTl, kThr, kK>;
    const int64_t k = k0 + (tid % S::kChunks) * 8;
#pragma unroll
    for (int i = 0; i < S::kPieces; ++i) {
        const int64_t row = min((int64_t)(r0 + tid / S::kChunks + S::kRowsPerPass * i), n - 1);
        v[i] = *reinterpret_cast<const half8*>(X + row * ldx + k);
    }
}

// The last, partial slab (or any slab of an unaligned X): element loads,
// tokens past ntok read as zero.
template <int kTl, int kThr, int kK>
__device__ __forceinline__ void fetch_tail(SlabRegs<kTl, kThr, kK>& v, const half_t* __restrict__ X, int64_t n,
                                           int64_t ldx, int64_t ntok, int r0, int64_t k0, int tid) {
    using S = Slab<kTl, kThr, kK>;
    const int64_t k = k0 + (tid % S::kChunks) * 8;
#pragma unroll
    for (int i = 0; i < S::kPieces; ++i) {
        const int64_t row = min((int64_t)(r0 + tid / S::kChunks + S::kRowsPerPass * i), n - 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = (k + e < ntok) ? X[row * ldx + k + e] : (half_t)0;
    }
}

template <int kTl, int kThr, int kK>
__device__ __forceinline__ void stash_slab(const SlabRegs<kTl, kThr, kK>& v, half_t* S_, int tid) {
    using S = Slab<kTl, kThr, kK>;
    const int kk = (tid % S::kChunks) * 8;
#pragma unroll
    for (int i = 0; i < S::kPieces; ++i)
        *reinterpret_cast<half8*>(&S_[(tid / S::kChunks + S::kRowsPerPass * i) * S::kLd + kk]) = v[i];
}

constexpr int kKf16 = 32;    // tokens per slab
constexpr int kDepthf16 = 2;  // slabs in flight per thread
// Layers with at least 16 tiles of 256 per side (d_in > 3840) take wide
// tiles; narrower ones the 128x128 tiles of four waves (41 KB of LDS, two
// workgroups per CU).  Among wide layers, those with at least two rounds of
// 256x256 tiles per CU take those, on 16 waves of one 64x64 quarter each
// (half the X bytes per product of 128x128 tiles, four waves per SIMD, 80 KB
// of LDS); the others the warp-specialised 192x192 kernel below, whose 253
// tiles at d_in = 4096 fill the chip where 136 tiles of 256 would not.
// Measured per 2048-token chunk: d_in = 4096, 54 against 75 us; d_in =
// 11008, 371 against 525 us.
constexpr int kWideTile = 256, kWideThreads = 1024, kWideMinT = 16, kWideMinRounds = 2;

// Slabs below nfull take the unconditional path; the rest (at most the last
// one, or all when X is unaligned) the element path.  Diagonal tiles load
// their one panel twice so that every tile issues the same loads.  The slab
// loop runs in two parts: a steady part in which every fetch is a full slab
// (so the compiler can count the loads in flight and wait only for the
// oldest set), and a generic part for the last slabs.
template <int kTl, int kThr, int kK, int kDepth>
__global__ __launch_bounds__(kThr, kThr == kThreads ? 2 : 1) void hessian_f16_kernel(float* __restrict__ H, int64_t n,
                                                                 const half_t* __restrict__ X, int64_t ldx,
                                                                 int64_t ntok, int64_t nfull, int T,
                                                                 int per_xcd, int set, const XChunks xc, int spc) {
    using S = Slab<kTl, kThr, kK>;
    constexpr int kWg = kTl / 64;  // computing waves per tile dimension (further waves only load)
    __shared__ half_t As[2][kTl * S::kLd];
    __shared__ half_t Bs[2][kTl * S::kLd];
    const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (t >= T * (T + 1) / 2) return;
    int I, J;
    tile_of_super(t, T, I, J);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w / kWg, wj = w % kWg;
    // waves past kWg^2 only load; on a diagonal tile the quarters above the
    // diagonal are skipped
    const bool active = w < kWg * kWg && !(I == J && wi < wj);
    const int rA = I * kTl, rB = J * kTl;

    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    const int64_t nslab = (ntok + kK - 1) / kK;
    SlabRegs<kTl, kThr, kK> ra[kDepth], rb[kDepth];

    // full slab f: slab f % spc of chunk f / spc (with several chunks)
    auto full = [&](SlabRegs<kTl, kThr, kK>& va, SlabRegs<kTl, kThr, kK>& vb, int64_t f) {
        const half_t* Xc = X;
        int64_t k0 = f * kK;
        if (spc) {
            const int c = (int)f / spc;
            Xc = xc.p[c];
            k0 = (f - (int64_t)c * spc) * kK;
        }
        fetch_full<kTl, kThr, kK>(va, Xc, n, ldx, rA, k0, tid);
        fetch_full<kTl, kThr, kK>(vb, Xc, n, ldx, rB, k0, tid);
    };
    auto fetch = [&](SlabRegs<kTl, kThr, kK>& va, SlabRegs<kTl, kThr, kK>& vb, int64_t f) {
        if (f < nfull) {
            full(va, vb, f);
        } else if (f < nslab) {
            fetch_tail<kTl, kThr, kK>(va, X, n, ldx, ntok, rA, f * kK, tid);
            fetch_tail<kTl, kThr, kK>(vb, X, n, ldx, ntok, rB, f * kK, tid);
        }
    };
    // stash slab sl from its registers, then (after the barrier) the MFMAs;
    // buffer sl&1 was last read by slab sl-2, which every wave finished
    // before the previous barrier
    auto stash = [&](const SlabRegs<kTl, kThr, kK>& va, const SlabRegs<kTl, kThr, kK>& vb, int64_t sl) {
        stash_slab<kTl, kThr, kK>(va, As[sl & 1], tid);
        stash_slab<kTl, kThr, kK>(vb, Bs[sl & 1], tid);
        __syncthreads();
    };
    auto compute = [&](int64_t sl) {
        if (!active) return;
        const half_t* Ap = As[sl & 1];
        const half_t* Bp = Bs[sl & 1];
        half8 a[kK / 16][2], b[kK / 16][2];
#pragma unroll
        for (int ks = 0; ks < kK / 16; ++ks) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
                a[ks][m] = *reinterpret_cast<const half8*>(
                    &Ap[(wi * 64 + 32 * m + (lane & 31)) * S::kLd + 16 * ks + 8 * (lane >> 5)]);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                b[ks][q] = *reinterpret_cast<const half8*>(
                    &Bp[(wj * 64 + 32 * q + (lane & 31)) * S::kLd + 16 * ks + 8 * (lane >> 5)]);
        }
#pragma unroll
        for (int ks = 0; ks < kK / 16; ++ks)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x16_f16(a[ks][m], b[ks][q], acc[m][q]);
    };

    // steady part: slabs [0, nsteady), every fetch (slab sl + kDepth) full;
    // its first fetches are unconditional too, so that on entry the compiler
    // sees exactly kDepth full sets of loads in flight
    const int64_t nsteady = nfull > kDepth ? ((nfull - kDepth) / kDepth) * kDepth : 0;
    int64_t s0 = 0;
    if (nsteady > 0) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            full(ra[d], rb[d], d);
            __builtin_amdgcn_sched_barrier(0);  // issue the sets in slab order
        }
        for (; s0 < nsteady; s0 += kDepth) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int64_t sl = s0 + d;
                stash(ra[d], rb[d], sl);
                full(ra[d], rb[d], sl + kDepth);
                compute(sl);
            }
        }
    } else {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) fetch(ra[d], rb[d], d);
    }
    // generic part: the last slabs
    for (; s0 < nslab; s0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int64_t sl = s0 + d;
            if (sl >= nslab) break;
            stash(ra[d], rb[d], sl);
            fetch(ra[d], rb[d], sl + kDepth);
            compute(sl);
        }
    }
    if (active) {
        if (set) store_quarter<true>(H, n, rA + wi * 64, rB + wj * 64, acc, lane);
        else store_quarter<false>(H, n, rA + wi * 64, rB + wj * 64, acc, lane);
    }
}

// ---------------------------------------------------------------------------
// float16 inputs, wide layers: 192x192 tiles, warp-specialised.
//
// Waves 0..8 each own a 64x64 quarter and only read LDS and issue MFMAs;
// waves 9..11 only load X and write the slabs into LDS, one slab ahead of
// the compute waves, so that the LDS writes of slab s+1 overlap the products
// of slab s (measured at d_in = 4096, 2048 tokens: 41.7 against 47.5 us for
// the loop when every wave both loads and computes).  64-token slabs, two LDS
// buffers, one barrier per slab: buffer (s+1)&1 is written after the barrier
// that ends slab s-1, whose readers have all finished with it by then.  The
// loaders hold one slab in registers beyond the one they write (a second
// measured no faster at 64 tokens per slab).
// ---------------------------------------------------------------------------
constexpr int kWsTile = 192, kWsK = 64, kWsDepth = 1;
constexpr int kWsCompute = 9, kWsLoaders = 3, kWsThreads = (kWsCompute + kWsLoaders) * 64;

// Loader side: thread lt of the 192 loader threads moves kWsPieces 16-byte
// pieces of the 384 x 64 slab (rows 0..191 of panel I, then 192..383 of
// panel J): piece i is row lt / 8 + 24 i, tokens (lt % 8) * 8 .. + 8.
constexpr int kWsChunks = kWsK / 8;
constexpr int kWsPieces = 2 * kWsTile * kWsChunks / (kWsLoaders * 64);
constexpr int kWsRowsPerPass = kWsLoaders * 64 / kWsChunks;
constexpr int kWsLd = kWsK + 8;  // padded LDS row (halves): conflict-free 16-byte MFMA operand reads
static_assert(kWsPieces * kWsRowsPerPass == 2 * kWsTile && kWsPieces % 2 == 0, "loader pieces cover both panels");

__global__ __launch_bounds__(kWsThreads, 1) void hessian_f16_ws_kernel(float* __restrict__ H, int64_t n,
                                                                       const half_t* __restrict__ X, int64_t ldx,
                                                                       int64_t ntok, int64_t nfull, int T,
                                                                       int per_xcd, int set, const XChunks xc, int spc) {
    __shared__ half_t As[2][kWsTile * kWsLd];
    __shared__ half_t Bs[2][kWsTile * kWsLd];
    const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (t >= T * (T + 1) / 2) return;
    int I, J;
    tile_of_super(t, T, I, J);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rA = I * kWsTile, rB = J * kWsTile;
    const int64_t nslab = (ntok + kWsK - 1) / kWsK;

    if (w >= kWsCompute) {
        const int lt = tid - kWsCompute * 64;
        const int chunk = lt % kWsChunks;
        // pieces 0..kWsPieces/2-1 lie in panel I, the rest in panel J (row
        // lt / 8 + 24 i < 192 exactly for i < 8)
        constexpr int kHalf = kWsPieces / 2;
        // byte offset of each piece (clamped row, first token of the piece)
        // from the first token of its slab: a full slab's loads take a
        // wave-uniform base plus these 32-bit offsets, with no per-load
        // 64-bit address arithmetic (the launcher checks that they fit)
        unsigned voff[kWsPieces];
        const int dst0 = (lt / kWsChunks) * kWsLd + chunk * 8;
#pragma unroll
        for (int i = 0; i < kWsPieces; ++i) {
            const int rr = lt / kWsChunks + kWsRowsPerPass * (i % kHalf);
            // rows past n are clamped to row n-1: they feed only accumulator
            // entries that are never stored
            const int64_t row = min((int64_t)((i < kHalf ? rA : rB) + rr), n - 1);
            voff[i] = (unsigned)((row * ldx + chunk * 8) * 2);
        }
        // first element of piece i's row
        auto rowp = [&](int i) {
            unsigned o = voff[i];
            asm volatile("" : "+v"(o));  // formed at each use, not kept as sixteen 64-bit pointers
            return reinterpret_cast<const half_t*>(reinterpret_cast<const char*>(X) + o) - chunk * 8;
        };
        half8 v[kWsDepth][kWsPieces];
        // a full slab: one unconditional 16-byte load per piece
        auto fetch_full_ws = [&](half8(&x)[kWsPieces], int64_t f) {
            // slab f % spc of chunk f / spc (with several chunks)
            const half_t* Xc = X;
            int64_t lf = f;
            if (spc) {
                const int c = (int)f / spc;
                Xc = xc.p[c];
                lf = f - (int64_t)c * spc;
            }
            const char* base = reinterpret_cast<const char*>(Xc + lf * kWsK);
#pragma unroll
            for (int i = 0; i < kWsPieces; ++i) x[i] = *reinterpret_cast<const half8*>(base + voff[i]);
        };
        // any slab: full ones as above, the partial last one (or every slab of
        // an unaligned X) by element loads with tokens past ntok read as zero;
        // slabs past the last are not loaded
        auto fetch = [&](half8(&x)[kWsPieces], int64_t f) {
            if (f < nfull) {
                fetch_full_ws(x, f);
            } else if (f < nslab) {
                // every element load is unconditional, from a token index
                // clamped to ntok-1, and the value past ntok replaced by zero
                // afterwards (a load under a branch would be waited for there)
                const int64_t k = f * kWsK + chunk * 8;
#pragma unroll
                for (int i = 0; i < kWsPieces; ++i) {
                    const half_t* p = rowp(i);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const half_t h = p[min(k + e, ntok - 1)];
                        x[i][e] = (k + e < ntok) ? h : (half_t)0;
                    }
                }
            }
        };
        auto put = [&](const half8(&x)[kWsPieces], int b) {
#pragma unroll
            for (int i = 0; i < kWsPieces; ++i)
                *reinterpret_cast<half8*>(&(i < kHalf ? As[b] : Bs[b])[dst0 + kWsRowsPerPass * (i % kHalf) * kWsLd]) = x[i];
        };
        // steady part: iterations whose refetch (slab sl + 1 + depth) is full,
        // entered with exactly kWsDepth full sets in flight so that each LDS
        // write waits only for the oldest set
        const int64_t lim = nfull - 1 - kWsDepth;
        const int64_t nsteady = lim > 0 ? (lim / kWsDepth) * kWsDepth : 0;
        if (nsteady > 0) {
#pragma unroll
            for (int d = 0; d < kWsDepth; ++d) {
                fetch_full_ws(v[d], d);
                __builtin_amdgcn_sched_barrier(0);
            }
            put(v[0], 0);
            fetch_full_ws(v[0], kWsDepth);
        } else {
#pragma unroll
            for (int d = 0; d < kWsDepth; ++d) fetch(v[d], d);
            put(v[0], 0);
            fetch(v[0], kWsDepth);
        }
        __syncthreads();
        // iteration sl writes slab sl+1 (held in set (sl+1) % depth) and
        // refills that set with slab sl+1+depth; one barrier per iteration
        int64_t s0 = 0;
        for (; s0 < nsteady; s0 += kWsDepth) {
#pragma unroll
            for (int d = 0; d < kWsDepth; ++d) {
                const int64_t sl = s0 + d;
                const int dn = (d + 1) % kWsDepth;
                put(v[dn], (int)((sl + 1) & 1));
                fetch_full_ws(v[dn], sl + 1 + kWsDepth);
                __syncthreads();
            }
        }
        for (; s0 < nslab; s0 += kWsDepth) {
#pragma unroll
            for (int d = 0; d < kWsDepth; ++d) {
                const int64_t sl = s0 + d;
                if (sl >= nslab) break;
                const int dn = (d + 1) % kWsDepth;
                if (sl + 1 < nslab) put(v[dn], (int)((sl + 1) & 1));
                fetch(v[dn], sl + 1 + kWsDepth);
                __syncthreads();
            }
        }
        return;
    }

    // compute waves: quarter (wi, wj) of the tile; on a diagonal tile the
    // quarters above the diagonal are skipped (their waves still take every
    // barrier)
    const int wi = w / 3, wj = w % 3;
    const bool active = !(I == J && wi < wj);
    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};
    const int offA = (wi * 64 + (lane & 31)) * kWsLd + 8 * (lane >> 5);
    const int offB = (wj * 64 + (lane & 31)) * kWsLd + 8 * (lane >> 5);
    __syncthreads();
    for (int64_t sl = 0; sl < nslab; ++sl) {
        if (active) {
            const half_t* Ap = As[sl & 1] + offA;
            const half_t* Bp = Bs[sl & 1] + offB;
#pragma unroll
            for (int ks = 0; ks < kWsK / 16; ++ks) {
                const half8 a0 = *reinterpret_cast<const half8*>(Ap + 16 * ks);
                const half8 a1 = *reinterpret_cast<const half8*>(Ap + 32 * kWsLd + 16 * ks);
                const half8 b0 = *reinterpret_cast<const half8*>(Bp + 16 * ks);
                const half8 b1 = *reinterpret_cast<const half8*>(Bp + 32 * kWsLd + 16 * ks);
                acc[0][0] = mfma32x32x16_f16(a0, b0, acc[0][0]);
                acc[0][1] = mfma32x32x16_f16(a0, b1, acc[0][1]);
                acc[1][0] = mfma32x32x16_f16(a1, b0, acc[1][0]);
                acc[1][1] = mfma32x32x16_f16(a1, b1, acc[1][1]);
            }
        }
        __syncthreads();
    }
    if (active) {
        if (set) store_quarter<true>(H, n, rA + wi * 64, rB + wj * 64, acc, lane);
        else store_quarter<false>(H, n, rA + wi * 64, rB + wj * 64, acc, lane);
    }
}

// ---------------------------------------------------------------------------
// float32 inputs
// ---------------------------------------------------------------------------
constexpr int kK32 = 32;
constexpr int kLd32 = kK32 + 4;

template <bool kVec>
__device__ __forceinline__ void load_slab_f32(float (*S)[kLd32], const float* __restrict__ X, int64_t n,
                                              int64_t ldx, int64_t ntok, int r0, int64_t k0, int tid) {
    const int kk = (tid & 7) * 4;
#pragma unroll
    for (int rr = 0; rr < kTile; rr += kThreads / 8) {
        int r = rr + (tid >> 3);
        int64_t row = r0 + r;
        int64_t k = k0 + kk;
        float4v v;
        if (kVec && row < n && k + 4 <= ntok) {
            v = *reinterpret_cast<const float4v*>(X + row * ldx + k);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (row < n && k + e < ntok) ? X[row * ldx + k + e] : 0.0f;
        }
        *reinterpret_cast<float4v*>(&S[r][kk]) = v;
    }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads, 2) void hessian_f32_kernel(float* __restrict__ H, int64_t n,
                                                              const float* __restrict__ X, int64_t ldx,
                                                              int64_t ntok, int set) {
    __shared__ float As[kTile][kLd32];
    __shared__ float Bs[kTile][kLd32];
    int I, J;
    tile_of(blockIdx.x, I, J);
    const bool diag = (I == J);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const bool active = !(diag && wi < wj);
    float(*Bp)[kLd32] = diag ? As : Bs;

    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    for (int64_t k0 = 0; k0 < ntok; k0 += kK32) {
        load_slab_f32<kVec>(As, X, n, ldx, ntok, I * kTile, k0, tid);
        if (!diag) load_slab_f32<kVec>(Bs, X, n, ldx, ntok, J * kTile, k0, tid);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int ks = 0; ks < kK32; ks += 2) {
                float a[2], b[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) a[m] = As[wi * 64 + 32 * m + (lane & 31)][ks + (lane >> 5)];
#pragma unroll
                for (int q = 0; q < 2; ++q) b[q] = Bp[wj * 64 + 32 * q + (lane & 31)][ks + (lane >> 5)];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x2_f32(a[m], b[q], acc[m][q]);
            }
        }
        __syncthreads();
    }
    if (active) {
        if (set) store_quarter<true>(H, n, I * kTile + wi * 64, J * kTile + wj * 64, acc, lane);
        else store_quarter<false>(H, n, I * kTile + wi * 64, J * kTile + wj * 64, acc, lane);
    }
}

// Row r of H: columns 0..r set to zero (the lower triangle of an empty sum).
__global__ __launch_bounds__(256) void zero_lower_kernel(float* __restrict__ H, int64_t n) {
    const int64_t r = blockIdx.x;
    for (int64_t c = threadIdx.x; c <= r; c += blockDim.x) H[r * n + c] = 0.0f;
}

}  // namespace

namespace {

// One float16 launch over g chunks of ntok tokens each (g = 1: xc.p[0] with
// any ntok; g > 1: every chunk aligned with ntok a multiple of 64).
hipError_t launch_f16(float* H, int64_t n, const XChunks& xc, int g, int64_t ntok, int64_t ldx, bool vec, int set,
                      hipStream_t s) {
    TimedLaunch t(K_HESS_F16, s);
    const half_t* X = xc.p[0];
    const int64_t tot = ntok * g;
    const int64_t T = (n + kTile - 1) / kTile;
    const int64_t tiles = T * (T + 1) / 2;
    // full slabs take 16-byte loads when every row start is 16-byte aligned
    const int64_t nfull = vec ? tot / kKf16 : 0;
    const int spc = g > 1 ? (int)(ntok / kKf16) : 0;
    const int64_t Tw = (n + kWideTile - 1) / kWideTile;
    const int64_t tw_all = Tw * (Tw + 1) / 2;
    const int n_cu = device_cu_count();
    if (Tw >= kWideMinT && n_cu > 0 && tw_all >= (int64_t)kWideMinRounds * n_cu) {
        const int per_xcd = (int)((tw_all + kXcds - 1) / kXcds);
        GPTQ_LAUNCH(t, (hessian_f16_kernel<kWideTile, kWideThreads, kKf16, kDepthf16>),
                    dim3((unsigned)(per_xcd * kXcds)), dim3(kWideThreads), 0, s, H, n, X, ldx, tot, nfull, (int)Tw,
                    per_xcd, set, xc, spc);
    } else if (Tw >= kWideMinT && (n - 1) * ldx * 2 + 256 < ((int64_t)1 << 32)) {
        // (the warp-specialised kernel addresses X by 32-bit byte offsets
        // from each slab's first token)
        const int64_t Tm = (n + kWsTile - 1) / kWsTile;
        const int64_t nfull_ws = vec ? tot / kWsK : 0;
        const int spc_ws = g > 1 ? (int)(ntok / kWsK) : 0;
        const int per_xcd = (int)((Tm * (Tm + 1) / 2 + kXcds - 1) / kXcds);
        GPTQ_LAUNCH(t, hessian_f16_ws_kernel, dim3((unsigned)(per_xcd * kXcds)), dim3(kWsThreads), 0, s, H, n, X,
                    ldx, tot, nfull_ws, (int)Tm, per_xcd, set, xc, spc_ws);
    } else {
        const int per_xcd = (int)((tiles + kXcds - 1) / kXcds);
        GPTQ_LAUNCH(t, (hessian_f16_kernel<kTile, kThreads, kKf16, kDepthf16>), dim3((unsigned)(per_xcd * kXcds)),
                    dim3(kThreads), 0, s, H, n, X, ldx, tot, nfull, (int)T, per_xcd, set, xc, spc);
    }
    return hipGetLastError();
}

hipError_t launch_one(float* H, int64_t n, const void* X, int x_is_f16, int64_t ntok, int64_t ldx, int set,
                      hipStream_t s) {
    if (ntok == 0) {
        if (!set) return hipSuccess;
        // H = 2 X X^T with no tokens: the lower triangle becomes zero
        TimedLaunch t(x_is_f16 ? K_HESS_F16 : K_HESS_F32, s);
        GPTQ_LAUNCH(t, zero_lower_kernel, dim3((unsigned)n), dim3(256), 0, s, H, n);
        return hipGetLastError();
    }
    const uintptr_t addr = reinterpret_cast<uintptr_t>(X);
    if (x_is_f16) {
        XChunks xc{};
        xc.p[0] = static_cast<const half_t*>(X);
        return launch_f16(H, n, xc, 1, ntok, ldx, (addr % 16 == 0) && (ldx % 8 == 0), set, s);
    }
    const int64_t T = (n + kTile - 1) / kTile;
    const int64_t tiles = T * (T + 1) / 2;
    TimedLaunch t(K_HESS_F32, s);
    const bool vec = (addr % 16 == 0) && (ldx % 4 == 0);
    if (vec)
        GPTQ_LAUNCH(t, hessian_f32_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, s, H, n,
                    static_cast<const float*>(X), ldx, ntok, set);
    else
        GPTQ_LAUNCH(t, hessian_f32_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, s, H, n,
                    static_cast<const float*>(X), ldx, ntok, set);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hessian(float* H, int64_t n, const void* const* Xs, int64_t nchunks, int x_is_f16, int64_t ntok,
                          int64_t ldx, int set, hipStream_t s) {
    if (n == 0 || nchunks <= 0) return hipSuccess;
    // several float16 chunks, each 16-byte aligned with whole 64-token slabs:
    // up to kMaxChunks of them summed in one launch, with one add into H
    bool batch = nchunks > 1 && x_is_f16 && ntok > 0 && ntok % 64 == 0 && ldx % 8 == 0 &&
                 ntok * kMaxChunks / kKf16 < ((int64_t)1 << 31);
    for (int64_t c = 0; batch && c < nchunks; ++c) batch = reinterpret_cast<uintptr_t>(Xs[c]) % 16 == 0;
    if (!batch) {
        for (int64_t c = 0; c < nchunks; ++c) {
            const hipError_t e = launch_one(H, n, Xs[c], x_is_f16, ntok, ldx, c == 0 ? set : 0, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    for (int64_t c0 = 0; c0 < nchunks; c0 += kMaxChunks) {
        const int g = (int)std::min<int64_t>(kMaxChunks, nchunks - c0);
        XChunks xc{};
        for (int i = 0; i < g; ++i) xc.p[i] = static_cast<const half_t*>(Xs[c0 + i]);
        const hipError_t e = g == 1 ? launch_one(H, n, xc.p[0], 1, ntok, ldx, c0 == 0 ? set : 0, s)
                                    : launch_f16(H, n, xc, g, ntok, ldx, true, c0 == 0 ? set : 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gptq
