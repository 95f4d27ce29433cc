// ltopk_kernels.hip -- top-k index selection for CSA on MI355X (gfx950, wave64).
//
// The selection (per row: the first min(k, |V|) valid positions by score,
// highest first, lower index first among equal scores) is the indexer top-k
// of DeepSeek-V4's compressed sparse attention: k = 512 per index-source layer,
// 2048 eight-position blocks for the shared-candidate layer ("SGLang 与 Miles 为
// DeepSeek-V4.1 提供首日支持", xhh.club, Q&A on cross-layer sharing). The talk
// notes on devpress.csdn.net (section 3.2) time it at a 1M-token context, batch
// size 1, and the AICon 2026 Shenzhen speaker page (aicon.infoq.cn, outline
// 三.2) describes their kernel as per-block histograms of a sharded row merged
// inside a thread-block cluster. CDNA4 has no clusters and LDS is private to a
// workgroup, so this file merges histograms through agent-scope atomics in a
// small global workspace instead (see the split kernel).
//
// Method used here (own design):
//   * every score becomes an order-preserving 32-bit key (integer ops only);
//     key 0 marks "no element", NaN maps to 1, -0.0 maps to +0.0's key;
//   * the pair (key, ~index) is a 64-bit composite that is unique per
//     position, so "top-m composites" is exactly the selection rule, ties
//     included, and no step depends on the order elements arrive in;
//   * an MSB-first radix select over the composite finds a prefix P at depth D
//     such that the elements whose D-digit prefix is >= P are exactly the
//     m selected ones (digits of 12/10/10 bits over the key, 11/11/10 over the
//     inverted index; most rows stop after one or two key digits);
//   * digit histograms live in LDS; wave64 shuffles build the block scans.
//
// Kernels:
//   split_kernel  : one row over S workgroups (keys held in VGPRs). S == 1 is
//                   fully local. S > 1 merges each digit histogram through
//                   global counters, meets at a per-row barrier (all S
//                   workgroups are co-resident: the host never launches more
//                   than fit at once), funnels the elements of the threshold
//                   bin to a global candidate list, and the last workgroup to
//                   finish (ticket counter) selects among them in LDS and
//                   returns the workspace to zero. Batch size 1 and decode.
//   stream_kernel : one workgroup per row reads the row once from HBM with
//                   non-temporal 16-byte loads, admits only elements that beat
//                   the current k-th best (a running threshold), keeps them in
//                   an LDS buffer and compacts it by radix select when it
//                   fills. Causal prefill (thousands of long rows).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "ltopk.h"
#include "ltopk_debug.h"

namespace ltk {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kCap = 4096;          // largest threshold bin funnelled to one workgroup
constexpr int kMaxSplitRows = 1024; // rows whose workspace one call may need at once

// ------------------------------------------------------------------ keys

// Order-preserving map from fp32 bits to an unsigned key: a larger key is a
// higher score. -0.0 gets +0.0's key, every NaN gets 1 (below -inf, whose key
// is 0x007FFFFF), and 0 is left free to mean "no element".
__device__ __forceinline__ uint32_t score_key(uint32_t u)
{
    uint32_t flip = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
    uint32_t key = u ^ flip;
    key = (u == 0x80000000u) ? 0x80000000u : key;
    key = ((u & 0x7fffffffu) > 0x7f800000u) ? 1u : key;
    return key;
}

__device__ __forceinline__ uint64_t comp(uint32_t key, uint32_t nid)
{
    return ((uint64_t)key << 32) | nid;
}

// Prefix of a composite: its bits at and above `s` (s == 64: empty prefix).
__device__ __forceinline__ uint64_t pfx(uint64_t c, int s)
{
    return s >= 64 ? 0ull : (c >> s);
}

// Digit schedules over the 64-bit composite. shift(d) is the lowest bit of the
// prefix fixed by the first d digits; digit d occupies [shift(d+1), shift(d)).
struct Sched12 { // first digit 12 bits: 4096-bin histograms
    static __device__ __forceinline__ int width(int d)
    {
        return d == 0 ? 12 : (d == 1 || d == 2 || d == 5) ? 10 : 11;
    }
    static __device__ __forceinline__ int shift(int d)
    {
        switch (d) {
        case 0: return 64;
        case 1: return 52;
        case 2: return 42;
        case 3: return 32;
        case 4: return 21;
        case 5: return 10;
        default: return 0;
        }
    }
    static constexpr int kMaxBins = 4096;
};

struct Sched11 { // first digit 11 bits: 2048-bin histograms
    static __device__ __forceinline__ int width(int d)
    {
        return (d == 2 || d == 5) ? 10 : 11;
    }
    static __device__ __forceinline__ int shift(int d)
    {
        switch (d) {
        case 0: return 64;
        case 1: return 53;
        case 2: return 42;
        case 3: return 32;
        case 4: return 21;
        case 5: return 10;
        default: return 0;
        }
    }
    static constexpr int kMaxBins = 2048;
};

// Where a radix select stands: the elements whose D-digit prefix is > P are
// selected (`above` of them); `cnt` elements have prefix == P and `need` of
// those still have to be taken. Exact when cnt == need.
struct SelState {
    int D;
    uint64_t P;
    uint32_t above;
    uint32_t cnt;
    uint32_t need;
};

// ---------------------------------------------------------- wave / block scans

__device__ __forceinline__ uint32_t wave_incl_prefix(uint32_t v)
{
    const int lane = __lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t t = __shfl_up(v, off, 64);
        if (lane >= off)
            v += t;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_suffix(uint32_t v)
{
    const int lane = __lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t t = __shfl_down(v, off, 64);
        if (lane + off < 64)
            v += t;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o < v ? o : v;
    }
    return v;
}

// Exclusive prefix sum of v over the block in thread order; total over all.
// tmp: LDS scratch of T/64 words.
template <int T>
__device__ __forceinline__ uint32_t block_excl_prefix(uint32_t v, uint32_t *tmp, uint32_t &total)
{
    constexpr int NW = T / 64;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    uint32_t inc = wave_incl_prefix(v);
    if (lane == 63)
        tmp[w] = inc;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        uint32_t x = tmp[i];
        off += (i < w) ? x : 0u;
        tot += x;
    }
    total = tot;
    __syncthreads();
    return off + inc - v;
}

struct BinHit {
    uint32_t bin, above, count, total;
};

// Threshold bin of an LDS histogram: the bin b with above(b) < need <=
// above(b) + hist[b], where above(b) counts the higher bins. Thread t owns the
// contiguous bins [t*per, t*per + per). Valid only if total >= need >= 1.
template <int T>
__device__ __forceinline__ BinHit block_find_bin(const uint32_t *hist, int nbins, uint32_t need,
                                                 uint32_t *tmp, uint32_t *res)
{
    constexpr int NW = T / 64;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int per = nbins >= T ? nbins / T : 1;
    const int lo = threadIdx.x * per;
    const int hi = lo + per < nbins ? lo + per : nbins;
    uint32_t s = 0;
    for (int b = lo; b < hi; ++b)
        s += hist[b];
    uint32_t inc = wave_incl_suffix(s);
    if (lane == 0)
        tmp[w] = inc;
    __syncthreads();
    uint32_t above = inc - s, total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        uint32_t x = tmp[i];
        above += (i > w) ? x : 0u;
        total += x;
    }
    if (s > 0 && above < need && above + s >= need) {
        uint32_t run = above;
        for (int b = hi - 1; b >= lo; --b) {
            uint32_t h = hist[b];
            if (run + h >= need) {
                res[0] = (uint32_t)b;
                res[1] = run;
                res[2] = h;
                break;
            }
            run += h;
        }
    }
    __syncthreads();
    BinHit r;
    r.bin = res[0];
    r.above = res[1];
    r.count = res[2];
    r.total = total;
    return r;
}

// Radix select over n composites held in LDS (all valid), continued from st
// until exact. hist must hold SCHED::kMaxBins words.
template <int T, class SCHED>
__device__ void lds_select(const uint32_t *ckey, const uint32_t *cnid, uint32_t n, SelState &st,
                           uint32_t *hist, uint32_t *tmp, uint32_t *res)
{
    while (st.cnt != st.need && st.D < 6) {
        const int W = SCHED::width(st.D);
        const int sp = SCHED::shift(st.D);
        const int sd = SCHED::shift(st.D + 1);
        const int nb = 1 << W;
        for (int b = threadIdx.x; b < nb; b += T)
            hist[b] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < n; i += T) {
            uint64_t c = comp(ckey[i], cnid[i]);
            if (pfx(c, sp) == st.P)
                atomicAdd(&hist[(uint32_t)(c >> sd) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        BinHit h = block_find_bin<T>(hist, nb, st.need, tmp, res);
        if (h.total < st.need)
            break; // inconsistent input (only after a timed-out barrier)
        st.above += h.above;
        st.need -= h.above;
        st.P = (st.P << W) | h.bin;
        st.cnt = h.count;
        st.D += 1;
    }
}

// ------------------------------------------------------------------ params

enum Mode { MODE_PLAIN = 0, MODE_BLOCKS = 1, MODE_CAND = 2 };

struct KParams {
    const float *scores;
    int64_t row_stride;
    const int32_t *lengths;
    int32_t n_max;
    int32_t k;           // k, or kb for the block stage
    const int32_t *cand; // [B, n_cand] block ids (MODE_CAND)
    int32_t n_cand;
    int32_t bs;          // block size (MODE_BLOCKS, MODE_CAND)
    int32_t row0;        // first row of this launch
    int32_t *out;        // [B, k]
    uint32_t *ws;        // workspace (split kernel, S > 1)
    uint32_t spin_limit;
};

// Per-row workspace layout (32-bit words). One global histogram per digit of
// Sched12, the counters, and the funnelled candidates as (key, ~index) pairs.
constexpr int kG0 = 0, kG1 = 4096, kG2 = 5120, kG3 = 6144, kG4 = 8192, kG5 = 10240;
constexpr int kCtr = 11264;
constexpr int kCtrArrive = kCtr + 0; // 6 words, one per digit
constexpr int kCtrTotal = kCtr + 6;
constexpr int kCtrOut = kCtr + 7;
constexpr int kCtrCand = kCtr + 8;
constexpr int kCtrTicket = kCtr + 9;
constexpr int kCtrStatus = kCtr + 10;
constexpr int kCandOff = kCtr + 64;
constexpr int kWsRowWords = kCandOff + 2 * kCap; // 19520 words = 78080 bytes

__device__ __forceinline__ int ghist_off(int d)
{
    switch (d) {
    case 0: return kG0;
    case 1: return kG1;
    case 2: return kG2;
    case 3: return kG3;
    case 4: return kG4;
    default: return kG5;
    }
}

__device__ __forceinline__ int32_t row_len(const KParams &p, int row)
{
    int32_t len = p.lengths[row];
    return len < 0 ? 0 : (len > p.n_max ? p.n_max : len);
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *a, uint32_t v)
{
    return __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t *a)
{
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All S workgroups of a row meet here. Counters are agent-scope atomics, so
// the workgroups may sit on different XCDs; the fences order each
// workgroup's histogram updates before its arrival and the others' updates
// before its reads. The wait is bounded: past spin_limit polls the status
// word is flagged and the workgroup moves on (results are then undefined, but
// every wave still finishes).
__device__ void row_barrier(uint32_t *ctr, uint32_t S, uint32_t spin_limit, uint32_t *status)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        atomic_add_agent(ctr, 1u);
        uint32_t it = 0;
        while (atomic_load_agent(ctr) < S) {
            __builtin_amdgcn_s_sleep(1);
            if (++it > spin_limit) {
                __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        __threadfence();
    }
    __syncthreads();
}

// ------------------------------------------------------------------ loaders

// Fill key[E] / nid[E] (nid = ~position) for this thread's share of the
// chunk of the virtual row starting at `base`. Absent elements get key 0.
template <int T, int E, int MODE>
struct Loader;

template <int T, int E>
struct Loader<T, E, MODE_PLAIN> {
    static_assert(E % 4 == 0, "plain rows load 4 scores per vector");
    static __device__ __forceinline__ void load(const KParams &p, int row, int32_t len, int64_t base,
                                                uint32_t (&key)[E], uint32_t (&nid)[E])
    {
        const float *x = p.scores + (int64_t)row * p.row_stride;
#pragma unroll
        for (int g = 0; g < E / 4; ++g) {
            const int64_t v0 = base + ((int64_t)g * T + threadIdx.x) * 4;
            f4 f = {0.f, 0.f, 0.f, 0.f};
            if (v0 < len)
                f = *reinterpret_cast<const f4 *>(x + v0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = v0 + j;
                key[4 * g + j] = (i < len) ? score_key(__float_as_uint(f[j])) : 0u;
                nid[4 * g + j] = ~(uint32_t)i;
            }
        }
    }
};

// Virtual element = a block of bs positions scored by its best valid key.
template <int T, int E>
struct Loader<T, E, MODE_BLOCKS> {
    static __device__ __forceinline__ void load(const KParams &p, int row, int32_t len, int64_t base,
                                                uint32_t (&key)[E], uint32_t (&nid)[E])
    {
        const float *x = p.scores + (int64_t)row * p.row_stride;
        const int64_t bs = p.bs;
        const int64_t nb = (len + bs - 1) / bs;
#pragma unroll
        for (int g = 0; g < E; ++g) {
            const int64_t blk = base + (int64_t)g * T + threadIdx.x;
            uint32_t best = 0;
            if (blk < nb) {
                const int64_t lo = blk * bs;
                if (bs == 8) {
                    f4 a = *reinterpret_cast<const f4 *>(x + lo);
                    f4 b = {0.f, 0.f, 0.f, 0.f};
                    if (lo + 4 < len)
                        b = *reinterpret_cast<const f4 *>(x + lo + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t ka = (lo + j < len) ? score_key(__float_as_uint(a[j])) : 0u;
                        uint32_t kb = (lo + 4 + j < len) ? score_key(__float_as_uint(b[j])) : 0u;
                        best = ka > best ? ka : best;
                        best = kb > best ? kb : best;
                    }
                } else {
                    const int64_t hi = lo + bs < len ? lo + bs : len;
                    for (int64_t i = lo; i < hi; ++i) {
                        uint32_t kk = score_key(__float_as_uint(x[i]));
                        best = kk > best ? kk : best;
                    }
                }
            }
            key[g] = best;
            nid[g] = ~(uint32_t)blk;
        }
    }
};

// Virtual element = slot s of the candidate list expanded to positions:
// slot s -> block cand[s / bs], offset s % bs.
template <int T, int E>
struct Loader<T, E, MODE_CAND> {
    static __device__ __forceinline__ void load(const KParams &p, int row, int32_t len, int64_t base,
                                                uint32_t (&key)[E], uint32_t (&nid)[E])
    {
        const float *x = p.scores + (int64_t)row * p.row_stride;
        const int32_t *cl = p.cand + (int64_t)row * p.n_cand;
        const int64_t bs = p.bs;
        if (bs == 8 && E % 8 == 0) {
#pragma unroll
            for (int g = 0; g < E / 8; ++g) {
                const int64_t slot = base / 8 + (int64_t)g * T + threadIdx.x;
                const int64_t b = slot < p.n_cand ? (int64_t)cl[slot] : -1;
                const int64_t lo = b * 8;
                f4 f0 = {0.f, 0.f, 0.f, 0.f}, f1 = {0.f, 0.f, 0.f, 0.f};
                const bool ok = b >= 0 && lo < len;
                if (ok) {
                    f0 = *reinterpret_cast<const f4 *>(x + lo);
                    if (lo + 4 < len)
                        f1 = *reinterpret_cast<const f4 *>(x + lo + 4);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    key[8 * g + j] = (ok && lo + j < len) ? score_key(__float_as_uint(f0[j])) : 0u;
                    key[8 * g + 4 + j] =
                        (ok && lo + 4 + j < len) ? score_key(__float_as_uint(f1[j])) : 0u;
                    nid[8 * g + j] = ~(uint32_t)(lo + j);
                    nid[8 * g + 4 + j] = ~(uint32_t)(lo + 4 + j);
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < E; ++g) {
                const int64_t v = base + (int64_t)g * T + threadIdx.x;
                const int64_t c = v / bs;
                const int64_t b = c < p.n_cand ? (int64_t)cl[c] : -1;
                const int64_t pos = b * bs + (v - c * bs);
                const bool ok = b >= 0 && pos < len;
                key[g] = ok ? score_key(__float_as_uint(x[pos])) : 0u;
                nid[g] = ~(uint32_t)pos;
            }
        }
    }
};

// Histogram of digit st.D over the register-resident elements whose prefix
// matches st.P. hist must be zeroed and the block synchronised by the caller.
template <class SCHED, int E>
__device__ __forceinline__ void regs_hist(const uint32_t (&key)[E], const uint32_t (&nid)[E],
                                          const SelState &st, uint32_t *hist)
{
    const int sp = SCHED::shift(st.D);
    const int sd = SCHED::shift(st.D + 1);
    const uint32_t mask = (1u << SCHED::width(st.D)) - 1u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint64_t c = comp(key[j], nid[j]);
        if (key[j] != 0u && pfx(c, sp) == st.P)
            atomicAdd(&hist[(uint32_t)(c >> sd) & mask], 1u);
    }
}

// ------------------------------------------------------------------ split kernel

template <int T, int E, int MODE>
__global__ __launch_bounds__(T) void split_kernel(KParams p)
{
    using SC = Sched12;
    constexpr int C = T * E;
    constexpr int NW = T / 64;
    __shared__ uint32_t hist[SC::kMaxBins];
    __shared__ uint32_t ckey[kCap];
    __shared__ uint32_t cnid[kCap];
    __shared__ uint32_t tmp[NW];
    __shared__ uint32_t res[4];
    __shared__ uint32_t bc[4];

    const int row = p.row0 + (int)blockIdx.y;
    const int wsrow = (int)blockIdx.y;
    const uint32_t S = gridDim.x;
    const int32_t len = row_len(p, row);
    const uint32_t k = (uint32_t)p.k;
    int32_t *out = p.out + (int64_t)row * p.k;

    uint32_t key[E], nid[E];
    Loader<T, E, MODE>::load(p, row, len, (int64_t)blockIdx.x * C, key, nid);

    uint32_t nvalid = 0;
#pragma unroll
    for (int j = 0; j < E; ++j)
        nvalid += key[j] != 0u ? 1u : 0u;

    SelState st;
    st.D = 0;
    st.P = 0;
    st.above = 0;

    if (S == 1) {
        // ---- whole row in this workgroup: exact radix select over registers
        uint32_t V;
        (void)block_excl_prefix<T>(nvalid, tmp, V);
        const uint32_t m = V < k ? V : k;
        st.cnt = V;
        st.need = m;
        while (st.cnt != st.need && st.D < 6) {
            const int nb = 1 << SC::width(st.D);
            for (int b = threadIdx.x; b < nb; b += T)
                hist[b] = 0;
            __syncthreads();
            regs_hist<SC>(key, nid, st, hist);
            __syncthreads();
            BinHit h = block_find_bin<T>(hist, nb, st.need, tmp, res);
            st.above += h.above;
            st.need -= h.above;
            st.P = (st.P << SC::width(st.D)) | h.bin;
            st.cnt = h.count;
            st.D += 1;
        }
        const int sD = SC::shift(st.D);
        uint32_t nsel = 0;
#pragma unroll
        for (int j = 0; j < E; ++j)
            nsel += (key[j] != 0u && pfx(comp(key[j], nid[j]), sD) >= st.P) ? 1u : 0u;
        uint32_t tot;
        uint32_t slot = block_excl_prefix<T>(nsel, tmp, tot);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (key[j] != 0u && pfx(comp(key[j], nid[j]), sD) >= st.P) {
                if (slot < k)
                    out[slot] = (int32_t)~nid[j];
                ++slot;
            }
        }
        for (uint32_t i = m + threadIdx.x; i < k; i += T)
            out[i] = -1;
        return;
    }

    // ---- row split over S workgroups
    uint32_t *ws = p.ws + (int64_t)wsrow * kWsRowWords;
    uint32_t m = 0;
    bool exact = false;
    int passes = 0; // global histograms written (to clear at the end)
    for (;;) {
        const int D = st.D;
        const int W = SC::width(D);
        const int nb = 1 << W;
        for (int b = threadIdx.x; b < nb; b += T)
            hist[b] = 0;
        __syncthreads();
        regs_hist<SC>(key, nid, st, hist);
        __syncthreads();
        // Bins below this workgroup's own need-th bin can never hold the
        // row's threshold, so only the higher bins are published.
        const uint32_t pr_need = D == 0 ? k : st.need;
        BinHit lh = block_find_bin<T>(hist, nb, pr_need, tmp, res);
        const uint32_t lg = lh.total >= pr_need ? lh.bin : 0u;
        uint32_t *G = ws + ghist_off(D);
        const int per = nb >= T ? nb / T : 1;
        const int blo = threadIdx.x * per;
        const int bhi = blo + per < nb ? blo + per : nb;
        for (int b = blo; b < bhi; ++b) {
            const uint32_t h = hist[b];
            if ((uint32_t)b >= lg && h != 0u)
                atomic_add_agent(&G[b], h);
        }
        if (D == 0 && threadIdx.x == 0 && lh.total != 0u)
            atomic_add_agent(&ws[kCtrTotal], lh.total);
        ++passes;
        row_barrier(&ws[kCtrArrive + D], S, p.spin_limit, &ws[kCtrStatus]);
        for (int b = blo; b < bhi; ++b)
            hist[b] = (uint32_t)b >= lg ? atomic_load_agent(&G[b]) : 0u;
        if (D == 0) {
            const uint32_t V = atomic_load_agent(&ws[kCtrTotal]);
            m = V < k ? V : k;
            st.cnt = V;
            st.need = m;
        }
        __syncthreads();
        if (st.cnt == st.need) {
            exact = true;
            break;
        }
        BinHit gh = block_find_bin<T>(hist, nb, st.need, tmp, res);
        if (gh.total < st.need) { // only after a timed-out barrier
            exact = true;
            break;
        }
        st.above += gh.above;
        st.need -= gh.above;
        st.P = (st.P << W) | gh.bin;
        st.cnt = gh.count;
        st.D += 1;
        if (st.cnt == st.need || st.D >= 6) {
            exact = true;
            break;
        }
        if (st.cnt <= (uint32_t)kCap)
            break;
    }

    // ---- funnel: emit the sure picks, publish the threshold bin
    const int sD = SC::shift(st.D);
    uint32_t nsel = 0, ncand = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (key[j] == 0u)
            continue;
        const uint64_t pre = pfx(comp(key[j], nid[j]), sD);
        if (exact ? pre >= st.P : pre > st.P)
            ++nsel;
        else if (pre == st.P)
            ++ncand;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_prefix<T>(nsel | (ncand << 16), tmp, tot);
    if (threadIdx.x == 0) {
        bc[0] = (tot & 0xffffu) ? atomic_add_agent(&ws[kCtrOut], tot & 0xffffu) : 0u;
        bc[1] = (tot >> 16) ? atomic_add_agent(&ws[kCtrCand], tot >> 16) : 0u;
    }
    __syncthreads();
    uint32_t so = bc[0] + (ex & 0xffffu);
    uint32_t co = bc[1] + (ex >> 16);
    uint2 *cbuf = reinterpret_cast<uint2 *>(ws + kCandOff);
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (key[j] == 0u)
            continue;
        const uint64_t pre = pfx(comp(key[j], nid[j]), sD);
        if (exact ? pre >= st.P : pre > st.P) {
            if (so < k)
                out[so] = (int32_t)~nid[j];
            ++so;
        } else if (pre == st.P) {
            if (co < (uint32_t)kCap)
                cbuf[co] = make_uint2(key[j], nid[j]);
            ++co;
        }
    }

    // ---- ticket: the last workgroup of the row finishes it
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t t = atomic_add_agent(&ws[kCtrTicket], 1u);
        bc[2] = (t == S - 1) ? 1u : 0u;
        __threadfence();
    }
    __syncthreads();
    if (bc[2] == 0u)
        return;

    // candidate entries written this call (cleared again below)
    uint32_t n_written = atomic_load_agent(&ws[kCtrCand]);
    n_written = n_written < (uint32_t)kCap ? n_written : (uint32_t)kCap;
    if (!exact) {
        uint32_t n = n_written;
        n = n < st.cnt ? n : st.cnt;
        n = n < (uint32_t)kCap ? n : (uint32_t)kCap;
        for (uint32_t i = threadIdx.x; i < n; i += T) {
            const uint2 e = cbuf[i];
            ckey[i] = e.x;
            cnid[i] = e.y;
        }
        if (threadIdx.x == 0)
            bc[3] = 0;
        __syncthreads();
        const uint32_t base_out = st.above;
        lds_select<T, SC>(ckey, cnid, n, st, hist, tmp, res);
        const int sF = SC::shift(st.D);
        for (uint32_t i = threadIdx.x; i < n; i += T) {
            if (pfx(comp(ckey[i], cnid[i]), sF) >= st.P) {
                const uint32_t s = base_out + atomicAdd(&bc[3], 1u);
                if (s < k)
                    out[s] = (int32_t)~cnid[i];
            }
        }
    }
    for (uint32_t i = m + threadIdx.x; i < k; i += T)
        out[i] = -1;

    // ---- return the workspace to zero for the next call
    __syncthreads();
    for (int d = 0; d < passes && d < 6; ++d) {
        const int nb = 1 << SC::width(d);
        uint32_t *G = ws + ghist_off(d);
        for (int b = threadIdx.x; b < nb; b += T)
            G[b] = 0u;
    }
    for (uint32_t i = threadIdx.x; i < n_written; i += T)
        cbuf[i] = make_uint2(0u, 0u);
    if (threadIdx.x < 16 && threadIdx.x != (kCtrStatus - kCtr))
        ws[kCtr + threadIdx.x] = 0u;
}

// ------------------------------------------------------------------ stream kernel

// One workgroup per row; the row is read once. Elements enter the LDS buffer
// only if their composite beats `thr`, the smallest composite kept by the last
// compaction (the running k-th best), so after a few sweeps almost nothing is
// admitted. Requires k <= kStreamBuf - SWEEP.
constexpr int kStreamBuf = 8192;

template <int T>
__global__ __launch_bounds__(T, 2) void stream_kernel(KParams p)
{
    using SC = Sched11;
    constexpr int EPT = 16;           // scores per thread per sweep (4 x 16 B)
    constexpr int U = EPT / 4;
    constexpr int SWEEP = T * EPT;    // 4096 for T = 256
    constexpr int CAPS = kStreamBuf - SWEEP;
    constexpr int NW = T / 64;
    constexpr int R = kStreamBuf / T; // buffer entries per thread when staged
    __shared__ uint32_t ckey[kStreamBuf];
    __shared__ uint32_t cnid[kStreamBuf];
    __shared__ uint32_t hist[SC::kMaxBins];
    __shared__ uint32_t tmp[NW];
    __shared__ uint32_t res[4];
    __shared__ uint32_t cnt3[3];
    __shared__ uint32_t slot_ctr;
    __shared__ uint64_t wmin[NW];

    const int row = p.row0 + (int)blockIdx.x;
    const int32_t len = row_len(p, row);
    const uint32_t k = (uint32_t)p.k;
    const float *x = p.scores + (int64_t)row * p.row_stride;
    int32_t *out = p.out + (int64_t)row * p.k;

    uint32_t thr_key = 0u, thr_nid = 0xffffffffu; // admit composite > thr
    uint32_t n_buf = 0;
    if (threadIdx.x == 0) {
        cnt3[0] = 0;
        cnt3[1] = 0;
        cnt3[2] = 0;
    }
    __syncthreads();

    const int nsw = (len + SWEEP - 1) / SWEEP;
    f4 cur[U], nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v0 = ((int64_t)u * T + threadIdx.x) * 4;
        cur[u] = f4{0.f, 0.f, 0.f, 0.f};
        if (v0 < len)
            cur[u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(x + v0));
    }
    for (int sw = 0; sw < nsw; ++sw) {
        const int64_t base = (int64_t)sw * SWEEP;
        if (sw + 1 < nsw) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v0 = base + SWEEP + ((int64_t)u * T + threadIdx.x) * 4;
                nxt[u] = f4{0.f, 0.f, 0.f, 0.f};
                if (v0 < len)
                    nxt[u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(x + v0));
            }
        }
        if (threadIdx.x == 0)
            cnt3[(sw + 1) % 3] = 0u;
        // admit
        uint32_t pass = 0; // bit e set: element e of this thread is admitted
        uint32_t kk[EPT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = base + ((int64_t)u * T + threadIdx.x) * 4 + j;
                const uint32_t key = (i < len) ? score_key(__float_as_uint(cur[u][j])) : 0u;
                const uint32_t nid = ~(uint32_t)i;
                kk[4 * u + j] = key;
                const bool ok = key > thr_key || (key == thr_key && nid > thr_nid);
                pass |= ok ? (1u << (4 * u + j)) : 0u;
            }
        }
        const uint64_t any = __ballot(pass != 0u);
        if (any) {
            const uint32_t c = __popc(pass);
            const uint32_t inc = wave_incl_prefix(c);
            const uint32_t wtot = __shfl(inc, 63, 64);
            uint32_t wbase = 0;
            if (__lane_id() == 0)
                wbase = atomicAdd(&cnt3[sw % 3], wtot);
            wbase = __shfl(wbase, 0, 64);
            uint32_t pos = n_buf + wbase + inc - c;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (pass & (1u << (4 * u + j))) {
                        if (pos < (uint32_t)kStreamBuf) {
                            ckey[pos] = kk[4 * u + j];
                            cnid[pos] = ~(uint32_t)(base + ((int64_t)u * T + threadIdx.x) * 4 + j);
                        }
                        ++pos;
                    }
                }
            }
        }
        __syncthreads();
        n_buf += cnt3[sw % 3];
        n_buf = n_buf < (uint32_t)kStreamBuf ? n_buf : (uint32_t)kStreamBuf;
        if (n_buf > (uint32_t)CAPS) {
            // ---- compaction: keep the top-k composites of the buffer
            SelState st;
            st.D = 0;
            st.P = 0;
            st.above = 0;
            st.cnt = n_buf;
            st.need = k;
            lds_select<T, SC>(ckey, cnid, n_buf, st, hist, tmp, res);
            const int sD = SC::shift(st.D);
            uint32_t rk[R], rn[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t i = (uint32_t)(r * T) + threadIdx.x;
                rk[r] = i < n_buf ? ckey[i] : 0u;
                rn[r] = i < n_buf ? cnid[i] : 0u;
            }
            if (threadIdx.x == 0)
                slot_ctr = 0;
            __syncthreads();
            uint64_t mn = ~0ull;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t c = comp(rk[r], rn[r]);
                if (rk[r] != 0u && pfx(c, sD) >= st.P) {
                    const uint32_t s = atomicAdd(&slot_ctr, 1u);
                    if (s < (uint32_t)kStreamBuf) {
                        ckey[s] = rk[r];
                        cnid[s] = rn[r];
                    }
                    mn = c < mn ? c : mn;
                }
            }
            mn = wave_min_u64(mn);
            if (__lane_id() == 0)
                wmin[threadIdx.x >> 6] = mn;
            __syncthreads();
            uint64_t t = ~0ull;
#pragma unroll
            for (int i = 0; i < NW; ++i)
                t = wmin[i] < t ? wmin[i] : t;
            n_buf = slot_ctr;
            thr_key = (uint32_t)(t >> 32);
            thr_nid = (uint32_t)t;
            __syncthreads();
        }
        if (sw + 1 < nsw) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                cur[u] = nxt[u];
        }
    }

    // ---- final selection over the buffer
    const uint32_t m = n_buf < k ? n_buf : k;
    SelState st;
    st.D = 0;
    st.P = 0;
    st.above = 0;
    st.cnt = n_buf;
    st.need = m;
    if (threadIdx.x == 0)
        slot_ctr = 0;
    __syncthreads();
    lds_select<T, SC>(ckey, cnid, n_buf, st, hist, tmp, res);
    const int sD = SC::shift(st.D);
    for (uint32_t i = threadIdx.x; i < n_buf; i += T) {
        if (m != 0u && pfx(comp(ckey[i], cnid[i]), sD) >= st.P) {
            const uint32_t s = atomicAdd(&slot_ctr, 1u);
            if (s < k)
                out[s] = (int32_t)~cnid[i];
        }
    }
    for (uint32_t i = m + threadIdx.x; i < k; i += T)
        out[i] = -1;
}

__global__ void empty_kernel() {}

// ------------------------------------------------------------------ host side

constexpr int kSplitT = 512;
constexpr int kPlainE = 8;  // 4096 scores per workgroup
constexpr int kBlocksE = 4; // 2048 blocks per workgroup
constexpr int kCandE = 8;   // 4096 candidate slots per workgroup
constexpr int kStreamT = 256;
constexpr uint32_t kDefaultSpin = 1u << 24;

struct KernelInfo {
    const void *fn;
    int occ;
};

struct DeviceInfo {
    bool ready;
    int cus;
    int occ_plain, occ_blocks, occ_cand;
};

static std::mutex g_mu;
static DeviceInfo g_dev[64];

static hipError_t device_info(DeviceInfo &out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.ready) {
        e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &d.occ_plain, reinterpret_cast<const void *>(split_kernel<kSplitT, kPlainE, MODE_PLAIN>),
            kSplitT, 0);
        if (e != hipSuccess)
            return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &d.occ_blocks,
            reinterpret_cast<const void *>(split_kernel<kSplitT, kBlocksE, MODE_BLOCKS>), kSplitT, 0);
        if (e != hipSuccess)
            return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &d.occ_cand, reinterpret_cast<const void *>(split_kernel<kSplitT, kCandE, MODE_CAND>),
            kSplitT, 0);
        if (e != hipSuccess)
            return e;
        d.ready = true;
    }
    out = d;
    return hipSuccess;
}

static uint32_t g_spin_limit = kDefaultSpin;
static int g_force_path = 0; // 0 auto, 1 split, 2 stream (rows without candidates)

template <int E, int MODE>
static lt_status launch_split(KParams p, int32_t B, int64_t vlen, int occ, int cus,
                              size_t ws_bytes, hipStream_t stream)
{
    constexpr int64_t C = (int64_t)kSplitT * E;
    const int64_t S = vlen > 0 ? (vlen + C - 1) / C : 1;
    if (S == 1) {
        // No inter-workgroup traffic: any number of rows in one launch.
        for (int32_t r0 = 0; r0 < B; r0 += 65535) {
            const int32_t rows = B - r0 < 65535 ? B - r0 : 65535;
            KParams q = p;
            q.row0 = r0;
            hipLaunchKernelGGL((split_kernel<kSplitT, E, MODE>), dim3(1, rows), dim3(kSplitT), 0,
                               stream, q);
        }
        return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
    }
    // Rows per launch: all workgroups of a launch must be resident together.
    int64_t cap = (int64_t)(occ > 0 ? occ : 1) * cus;
    int64_t rows_per = cap / S;
    if (rows_per < 1)
        return LT_EINVAL; // a single row would not fit on the device at once
    if (rows_per > kMaxSplitRows)
        rows_per = kMaxSplitRows;
    if (ws_bytes < (size_t)(rows_per < B ? rows_per : B) * kWsRowWords * 4 || p.ws == nullptr)
        return LT_ENOSPC;
    for (int32_t r0 = 0; r0 < B; r0 += (int32_t)rows_per) {
        const int32_t rows = (int32_t)(B - r0 < rows_per ? B - r0 : rows_per);
        KParams q = p;
        q.row0 = r0;
        hipLaunchKernelGGL((split_kernel<kSplitT, E, MODE>), dim3((unsigned)S, rows), dim3(kSplitT),
                           0, stream, q);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

static lt_status launch_stream(KParams p, int32_t B, hipStream_t stream)
{
    for (int32_t r0 = 0; r0 < B; r0 += 1 << 30) {
        KParams q = p;
        q.row0 = r0;
        const int32_t rows = B - r0;
        hipLaunchKernelGGL((stream_kernel<kStreamT>), dim3(rows), dim3(kStreamT), 0, stream, q);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

static lt_status validate_common(const float *scores, int64_t row_stride, const int32_t *lengths,
                                 int32_t B, int32_t n_max, int32_t k, const void *out)
{
    if (!scores || !lengths || !out)
        return LT_EINVAL;
    if (B < 0 || n_max < 0 || k < 1 || k > LT_K_MAX)
        return LT_EINVAL;
    if (row_stride < n_max || row_stride % 4 != 0)
        return LT_EINVAL;
    if (((uintptr_t)scores & 15u) != 0u)
        return LT_EINVAL;
    return LT_OK;
}

static lt_status check_ws(void *workspace)
{
    return ((uintptr_t)workspace & 15u) == 0u ? LT_OK : LT_EINVAL;
}

} // namespace ltk

using namespace ltk;

extern "C" {

size_t lt_topk_workspace_bytes(int32_t B, int32_t n_max, int32_t k)
{
    (void)k;
    if (B <= 0 || n_max <= 2048)
        return 0;
    const int64_t rows = B < kMaxSplitRows ? B : kMaxSplitRows;
    return (size_t)rows * kWsRowWords * 4u;
}

lt_status lt_topk_run(const float *scores, int64_t row_stride, const int32_t *lengths, int32_t B,
                      int32_t n_max, int32_t k, const lt_cand_t *cand, int32_t *out_idx,
                      void *workspace, size_t ws_bytes, lt_stream_t stream)
{
    lt_status st = validate_common(scores, row_stride, lengths, B, n_max, k, out_idx);
    if (st != LT_OK)
        return st;
    if (cand && (!cand->blocks || cand->n_blocks < 1 || cand->block_size < 1))
        return LT_EINVAL;
    if ((st = check_ws(workspace)) != LT_OK)
        return st;
    if (B == 0)
        return LT_OK;
    DeviceInfo d;
    if (device_info(d) != hipSuccess)
        return LT_EHIP;
    KParams p = {};
    p.scores = scores;
    p.row_stride = row_stride;
    p.lengths = lengths;
    p.n_max = n_max;
    p.k = k;
    p.out = out_idx;
    p.ws = static_cast<uint32_t *>(workspace);
    p.spin_limit = g_spin_limit;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (cand) {
        p.cand = cand->blocks;
        p.n_cand = cand->n_blocks;
        p.bs = cand->block_size;
        const int64_t vlen = (int64_t)cand->n_blocks * cand->block_size;
        return launch_split<kCandE, MODE_CAND>(p, B, vlen, d.occ_cand, d.cus, ws_bytes, s);
    }
    constexpr int64_t C = (int64_t)kSplitT * kPlainE;
    const int64_t S = n_max > 0 ? ((int64_t)n_max + C - 1) / C : 1;
    const int64_t cap = (int64_t)d.occ_plain * d.cus;
    bool use_split = S == 1 || ((int64_t)B * S <= cap && B <= kMaxSplitRows);
    if (g_force_path == 1)
        use_split = true;
    else if (g_force_path == 2)
        use_split = false;
    if (use_split)
        return launch_split<kPlainE, MODE_PLAIN>(p, B, n_max, d.occ_plain, d.cus, ws_bytes, s);
    return launch_stream(p, B, s);
}

lt_status lt_topk_blocks(const float *scores, int64_t row_stride, const int32_t *lengths, int32_t B,
                         int32_t n_max, int32_t block_size, int32_t kb, int32_t *out_blocks,
                         void *workspace, size_t ws_bytes, lt_stream_t stream)
{
    lt_status st = validate_common(scores, row_stride, lengths, B, n_max, kb, out_blocks);
    if (st != LT_OK)
        return st;
    if (block_size < 1)
        return LT_EINVAL;
    if ((st = check_ws(workspace)) != LT_OK)
        return st;
    if (B == 0)
        return LT_OK;
    DeviceInfo d;
    if (device_info(d) != hipSuccess)
        return LT_EHIP;
    KParams p = {};
    p.scores = scores;
    p.row_stride = row_stride;
    p.lengths = lengths;
    p.n_max = n_max;
    p.k = kb;
    p.bs = block_size;
    p.out = out_blocks;
    p.ws = static_cast<uint32_t *>(workspace);
    p.spin_limit = g_spin_limit;
    const int64_t vlen = ((int64_t)n_max + block_size - 1) / block_size;
    return launch_split<kBlocksE, MODE_BLOCKS>(p, B, vlen, d.occ_blocks, d.cus, ws_bytes,
                                               reinterpret_cast<hipStream_t>(stream));
}

int lt_debug_force_path(int path)
{
    const int prev = g_force_path;
    if (path >= 0 && path <= 2)
        g_force_path = path;
    return prev;
}

uint32_t lt_debug_set_spin_limit(uint32_t polls)
{
    const uint32_t prev = g_spin_limit;
    g_spin_limit = polls;
    return prev;
}

int lt_debug_empty_launch(int32_t grid_x, int32_t grid_y, int32_t block, void *stream)
{
    if (grid_x < 1 || grid_y < 1 || grid_y > 65535 || block < 1 || block > 1024)
        return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(grid_x, grid_y), dim3(block), 0,
                       reinterpret_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

size_t lt_debug_status_offset(int32_t row)
{
    return ((size_t)(row < 0 ? 0 : row) * kWsRowWords + kCtrStatus) * 4u;
}

const char *lt_status_str(lt_status status)
{
    switch (status) {
    case LT_OK: return "LT_OK: success";
    case LT_EINVAL: return "LT_EINVAL: invalid argument (nothing launched)";
    case LT_ENOSPC: return "LT_ENOSPC: workspace too small";
    case LT_EHIP: return "LT_EHIP: HIP runtime error at launch";
    default: return "unknown lt_status";
    }
}

} // extern "C"
