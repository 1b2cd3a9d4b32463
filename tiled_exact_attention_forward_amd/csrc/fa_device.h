// fa_device.h -- device-side building blocks shared by the forward and backward kernels
// (gfx950): fragment types and MFMA wrappers, LDS swizzles, the key-tile schedule of a query
// tile under each mask, the element mask, the direct HBM-to-LDS tile loads and the ring
// barrier. Included by one kernel file per translation unit (everything has internal
// linkage).
#pragma once
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace teaf {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) const char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;
// Mask id of the block-sparse path (layout of kSparseBlock x kSparseBlock tiles) and the
// largest number of key blocks a query block's list holds.
constexpr int kBlockSparse = kMaskBlockSparse, kSparseBlock = kBlockSparseEdge,
              kMaxKeyBlocks = kBlockSparseMaxKeyBlocks;


// Hardware hands consecutive workgroup ids to the 8 XCDs in turn. Map id w (of n) to a
// logical index so that each XCD receives one contiguous run of logical indices.
__device__ __forceinline__ int xcd_remap(int w, int n)
{
    const int per = n / kXcds, rem = n % kXcds;
    const int x = w % kXcds, idx = w / kXcds;
    return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

template <int MASK>
__device__ __forceinline__ bool key_visible(int ip, int j, int W, int G)
{
    if (MASK == 0 || MASK == kBlockSparse) return true;  // block sparse: decided per tile
    if (MASK == 1) return j <= ip;
    if (MASK == 3) return j >= ip - W && j <= ip + W;
    if (MASK == 4) return j <= ip || j < G;
    return j <= ip && (ip - j < W || j < G);
}

// Key tiles visible to query rows [q0, min(q0+BM, Nq)): [a0,a1) then [b0,b1), ascending.
struct TileRanges {
    int a0, a1, b0, b1;
};

template <int MASK, int BM, int BN>
__device__ __forceinline__ TileRanges visible_tiles(int q0, int Nq, int Nkv, int W, int G)
{
    TileRanges r{0, (Nkv + BN - 1) / BN, 0, 0};
    if (MASK == 0 || MASK == kBlockSparse) return r;
    const int delta = Nkv - Nq;
    if (MASK == 3) {  // band: from the first row's oldest key to the last row's newest key
        const int lo = max(0, q0 + delta - W);
        const int hi = min(Nkv - 1, min(q0 + BM, Nq) - 1 + delta + W);
        if (hi < lo) {
            r.a1 = 0;
            return r;
        }
        r.a0 = lo / BN;
        r.a1 = hi / BN + 1;
        return r;
    }
    if (MASK == 4) {  // prefix LM: the prefix and everything up to the last row
        const int last = min(Nkv - 1, max(min(q0 + BM, Nq) - 1 + delta, G - 1));
        r.a1 = last < 0 ? 0 : last / BN + 1;
        return r;
    }
    const int last = min(Nkv - 1, min(q0 + BM, Nq) - 1 + delta);  // newest visible key
    if (last < 0) {
        r.a1 = 0;
        return r;
    }
    const int t_end = last / BN + 1;
    r.a1 = t_end;
    if (MASK == 1) return r;
    const int first = max(0, q0 + delta - W + 1);  // oldest window key of the first row
    const int w_begin = first / BN;
    const int g_end = (min(G, last + 1) + BN - 1) / BN;
    if (g_end >= w_begin) return r;  // global tiles touch the window: one range
    r.a1 = g_end;
    r.b0 = w_begin;
    r.b1 = t_end;
    return r;
}

// Key-tile schedule of one query tile: the visible tiles, ordered so that the tiles every
// row of the tile sees completely ("interior": no mask, no tail) come first and the
// remaining visible tiles ("edge") last: two interior ranges, then the visible parts of the
// (up to three) gaps around them, one slot for every pairing of gap and visible range.
constexpr int kRanges = 8;
struct TileSchedule {
    int b[kRanges], e[kRanges];
    int interior, total;

    // Walks the schedule one tile at a time; work beyond an increment happens only when a
    // range ends.
    struct Cursor {
        int k, t, end;
    };
    __device__ __forceinline__ Cursor seek(int k) const
    {
        Cursor c{kRanges, 0, 0};
#pragma unroll
        for (int q = kRanges - 1; q >= 0; --q)
            if (q >= k && e[q] > b[q]) c = Cursor{q, b[q], e[q]};
        return c;
    }
    __device__ __forceinline__ Cursor begin() const { return seek(0); }
    __device__ __forceinline__ Cursor next(Cursor c) const
    {
        return c.t + 1 < c.end ? Cursor{c.k, c.t + 1, c.end} : seek(c.k + 1);
    }
    // The cursor at schedule position p (past the end: the end cursor, as seek gives).
    __device__ __forceinline__ Cursor at(int p) const
    {
        Cursor c{kRanges, 0, 0};
        int base = 0;
        bool found = false;
#pragma unroll
        for (int q = 0; q < kRanges; ++q) {
            const int n = e[q] - b[q];
            if (!found && p < base + n) {
                c = Cursor{q, b[q] + p - base, e[q]};
                found = true;
            }
            base += n;
        }
        return c;
    }
    // Tile at position p < interior: the interior ranges are ranges 0 and 1 (either may be
    // empty), so no walk over the ranges.
    __device__ __forceinline__ int interior_tile(int p) const
    {
        const int n0 = e[0] - b[0];
        return p < n0 ? b[0] + p : b[1] + (p - n0);
    }
};

__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

template <int MASK, int BM, int BN>
__device__ __forceinline__ TileSchedule make_schedule(int q0, int Nq, int Nkv, int W, int G)
{
    TileSchedule s;
#pragma unroll
    for (int k = 0; k < kRanges; ++k) s.b[k] = s.e[k] = 0;
    const TileRanges v = visible_tiles<MASK, BM, BN>(q0, Nq, Nkv, W, G);
    // interior ranges, judged for every row of the tile (padding rows included)
    const int delta = Nkv - Nq;
    const int ip0 = q0 + delta, ip1 = q0 + BM - 1 + delta;
    int lim = Nkv / BN;  // tiles without a key tail
    if (MASK == 1 || MASK == 2) lim = min(lim, max(0, floor_div(ip0 + 1, BN)));  // causal
    int i0b = 0, i0e = lim, i1b = 0, i1e = 0;
    if (MASK == 2) {
        const int gend = G / BN;                                   // all keys global
        const int wbeg = max(0, -floor_div(-(ip1 - W + 1), BN));   // in every row's window
        i0e = min(gend, lim);
        i1b = max(wbeg, i0e);
        i1e = lim;
        if (i1b >= i1e) i1b = i1e = 0;
    }
    if (MASK == 3) {  // keys every row sees: [ip1 - W, ip0 + W]
        i0b = max(0, -floor_div(-(ip1 - W), BN));
        i0e = min(lim, floor_div(ip0 + W + 1, BN));
    }
    if (MASK == 4)  // keys every row sees: the prefix and everything up to the first row
        i0e = min(lim, max(0, floor_div(max(G, ip0 + 1), BN)));
    if (i0e <= i0b) i0b = i0e = 0;
    s.b[0] = i0b; s.e[0] = i0e;
    s.b[1] = i1b; s.e[1] = i1e;
    s.interior = (i0e - i0b) + (i1e - i1b);
    // edge ranges: the gaps around the interior ranges, intersected with the visible ranges
    const int big = 0x3fffffff;
    const bool h0 = i0e > i0b, h1 = i1e > i1b;
    const int ga_b = 0, ga_e = h0 ? i0b : (h1 ? i1b : big);      // before the interior
    const int gb_b = h0 && h1 ? i0e : 0, gb_e = h0 && h1 ? i1b : 0;  // between the two
    const int gc_b = h1 ? i1e : (h0 ? i0e : 0), gc_e = h0 || h1 ? big : 0;  // after it
    auto put = [&s](int slot, int lo0, int hi0, int lo1, int hi1) {
        const int lo = max(lo0, lo1), hi = min(hi0, hi1);
        s.b[slot] = hi > lo ? lo : 0;
        s.e[slot] = hi > lo ? hi : 0;
    };
    put(2, ga_b, ga_e, v.a0, v.a1);
    put(3, ga_b, ga_e, v.b0, v.b1);
    put(4, gb_b, gb_e, v.a0, v.a1);
    put(5, gb_b, gb_e, v.b0, v.b1);
    put(6, gc_b, gc_e, v.a0, v.a1);
    put(7, gc_b, gc_e, v.b0, v.b1);
    s.total = 0;
#pragma unroll
    for (int q = 0; q < kRanges; ++q) s.total += s.e[q] - s.b[q];
    return s;
}

// Block-sparse lists: the indices b < n (n <= kMaxKeyBlocks) for which pred(b) holds, in
// ascending order, stored in LDS by the NW waves of a workgroup (ballot and popcount per wave,
// the wave counts combined through wcnt[NW] in LDS). Returns the number of entries, the same
// in every wave.
template <int NW, typename Pred>
__device__ __forceinline__ int compact_list(int *wcnt, uint16_t *list, int n, int tid, Pred pred)
{
    constexpr int CH = kMaxKeyBlocks / (64 * NW);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    bool f[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {  // every layout load first, one wait
        const int b = u * 64 * NW + tid;
        f[u] = b < n && pred(b);
    }
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
        if (u * 64 * NW >= n) break;
        const unsigned long long mk = __ballot(f[u]);
        if (lane == 0) wcnt[wave] = __popcll(mk);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int cw = wcnt[w];
            before += w < wave ? cw : 0;
            total += cw;
        }
        if (f[u])
            list[cnt + before + __popcll(mk & ((1ull << lane) - 1))] =
                (uint16_t)(u * 64 * NW + tid);
        cnt += total;
        __syncthreads();
    }
    return cnt;
}

// Key tiles of one query block under a block-sparse layout: lists the key blocks whose
// entries in lrow (nkb of them) are set, at `at` + 16 in LDS (wave counts at `at`), and sets
// the stream length ntl (position p holds key tile (kSparseBlock / BN) * list[p / (kSparseBlock
// / BN)] + p % (kSparseBlock / BN); only the final key block can have fewer tiles, and it
// comes last) and nint, the positions before the one tile with a key tail, if any.
template <int NW, int BN>
__device__ __forceinline__ void key_block_list(char *at, const uint8_t *lrow, int nkb, int Nkv,
                                               int tid, int &ntl, int &nint)
{
    constexpr int TPB = kSparseBlock / BN;
    uint16_t *list = (uint16_t *)(at + 16);
    const int n = compact_list<NW>((int *)at, list, nkb, tid, [&](int b) { return lrow[b] != 0; });
    ntl = nint = 0;
    if (n > 0) {
        const int lastb = __builtin_amdgcn_readfirstlane((int)list[n - 1]);
        const int all = (Nkv + BN - 1) / BN;
        ntl = TPB * (n - 1) + (lastb == nkb - 1 ? all - TPB * lastb : TPB);
        nint = ntl - (lastb == nkb - 1 && Nkv % BN != 0 ? 1 : 0);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum that propagates NaN; it needs no quieting of its inputs, so a chain of them maps to
// three-input maximum instructions.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Combine a value with the one held by lane ^ 32 (the other half of the wave) through a
// cross-half register swap, without a round trip through LDS.
__device__ __forceinline__ float half_swap_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
struct Ops16;

template <>
struct Ops16<__bf16> {
    static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ s16x8 pack8(float a0, float a1, float a2, float a3,
                                                  float a4, float a5, float a6, float a7)
    {
        bf16x8 r = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3,
                    (__bf16)a4, (__bf16)a5, (__bf16)a6, (__bf16)a7};
        return __builtin_bit_cast(s16x8, r);
    }
    static __device__ __forceinline__ s16x4 pack4(float a0, float a1, float a2, float a3)
    {
        bf16x4 r = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3};
        return __builtin_bit_cast(s16x4, r);
    }
};

template <>
struct Ops16<_Float16> {
    static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ s16x8 pack8(float a0, float a1, float a2, float a3,
                                                  float a4, float a5, float a6, float a7)
    {
        f16x8 r = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3,
                   (_Float16)a4, (_Float16)a5, (_Float16)a6, (_Float16)a7};
        return __builtin_bit_cast(s16x8, r);
    }
    static __device__ __forceinline__ s16x4 pack4(float a0, float a1, float a2, float a3)
    {
        f16x4 r = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3};
        return __builtin_bit_cast(s16x4, r);
    }
};

// Store a wave's 32 x D output tile (accumulator layout of the 32x32 MFMA: lane (g, i) holds
// 8-byte pieces of row i) as whole rows. Stored straight from the accumulator, each
// instruction would write 16 bytes of each of 32 rows; instead the tile is staged in LDS at
// st (32 rows of pitch D*2 + 16 bytes: 16-byte aligned, and the row-wise read-back is free
// of bank conflicts) and read back so that each store writes 64 / (D / 8) complete rows.
// Rows r with row0 + r >= nvalid are not stored; row r goes to out + (row0 + r) * rs.
// The wave reads back only what it wrote itself: LDS operations of one wave complete in
// order, so no barrier separates the writes from the reads.
template <typename T, int D>
__device__ __forceinline__ void store_rows_via_lds(char *st, const f32x16 (&acc)[D / 32],
                                                   float mul, int lane, uint16_t *out,
                                                   int row0, int nvalid, int rs)
{
    constexpr int OP = 2 * D + 16, CH = D / 8, RPI = 64 / CH;
    const int g = lane >> 5, li = lane & 31;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const s16x4 v4 = Ops16<T>::pack4(acc[db][4 * blk] * mul, acc[db][4 * blk + 1] * mul,
                                             acc[db][4 * blk + 2] * mul,
                                             acc[db][4 * blk + 3] * mul);
            *(s16x4 *)(st + li * OP + 2 * (db * 32 + 8 * blk + 4 * g)) = v4;
        }
    }
    const int rr = lane / CH, cc = lane % CH;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
        const int r = it * RPI + rr;
        const s16x8 v8 = *(const s16x8 *)(st + r * OP + 16 * cc);
        if (row0 + r < nvalid) *(s16x8 *)(out + (size_t)(row0 + r) * rs + 8 * cc) = v8;
    }
}

// ------------------------------------------------------------------ 16-bit kernel

// LDS tiles are unpadded rows with an XOR swizzle of the 16-byte chunks (an involution:
// the same function maps logical to physical and back). Chosen against the 64-bank LDS:
// a ds_read_b128 serves 16 lanes per cycle, here 16 consecutive K rows at one logical
// chunk; a ds_read_b64_tr_b16 serves 32 lanes, here 4 consecutive V rows x 64 bytes.
template <int D>
__device__ __forceinline__ int k_swz(int row, int chunk)
{
    return D == 128 ? chunk ^ (row & 15) : chunk ^ ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row, int chunk)
{
    return D == 128 ? chunk ^ (4 * (row & 3)) : chunk ^ (4 * ((row >> 1) & 1));
}

typedef __attribute__((address_space(3))) void lds_void;


// Each wave owns 32 query rows and walks 32-key tiles, software-pipelined: while the
// matrix cores form the scores of tile t+1, the vector unit turns the scores of tile t into
// probabilities; while they add P(t) V(t) into the accumulator, the vector unit sums P(t)
// and takes the row maximum of tile t+1. The instruction order is fixed with scheduling
// barriers. K and V tiles stream from HBM into a ring of NS LDS slots, NS - 2 tiles ahead of
// their first use.

template <int D, int NS, int NW_>
struct CfgSP {
    static constexpr int NW = NW_, BM = 32 * NW, BN = 32, NT = 64 * NW;
    static constexpr int ROWB = D * 2;                 // bytes of one K or V row
    static constexpr int TILEB = BN * ROWB;            // bytes of one K (or V) tile
    static constexpr int VREG = NS * TILEB;            // V ring starts after the K ring
    static constexpr int LDS_BYTES = 2 * NS * TILEB;
    static constexpr int CHUNKS = ROWB / 16;
    static constexpr int ROWS_PER_LOAD = 64 / CHUNKS;  // rows one wave-wide 16-byte load fills
    static constexpr int KL = TILEB / 1024;            // wave-wide loads per K (or V) tile
    static constexpr int LPW = 2 * KL / NW;            // loads per wave per tile (K and V)
    static_assert(LPW * NW == 2 * KL, "tile loads must split evenly over the waves");
    static constexpr int NKK = D / 16, NDB = D / 32;
    static constexpr int KPF = 3;                      // K fragment reads in flight
    static constexpr int VPF = 2;                      // V fragment read pairs in flight
};

// Wait until at most `newer` tiles' loads (LPW per tile, this wave's share) are still in
// flight; loads complete in issue order. vmcnt takes an immediate (6 bits, split over
// bits 3:0 and 15:14; expcnt and lgkmcnt left unconstrained), hence one case per count.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

template <int LPW, int K>
__device__ __forceinline__ void wait_tiles(int newer)
{
    static_assert(K * LPW < 64, "vmcnt field");
    if constexpr (K <= 0) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
        if (newer >= K)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(K * LPW));
        else
            wait_tiles<LPW, K - 1>(newer);
    }
}

// Workgroup barrier for the LDS ring: waits for this wave's LDS instructions only. The
// direct-to-LDS loads of tiles further ahead stay in flight (the compiler's fences would
// wait for every outstanding load, since those loads write LDS); their completion is
// awaited explicitly with wait_tiles before the barrier that publishes a tile. The empty
// asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void ring_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Direct HBM-to-LDS loads of this wave's share of the K and V tile that starts at key kv0.
// Load i of a tile (i < KL: K, else V) fills 1 KB, i.e. ROWS_PER_LOAD rows, of its LDS
// tile; wave w issues loads w, w + NW, ... off[u]: this lane's byte offset in the tile.
// Issue the loads of one K tile and one V tile (32 rows each) from HBM straight into LDS.
// kt and vt point at the tiles' first rows; rest is the number of valid bytes from there
// (the buffer range check returns zeros past it, so tail rows arrive as zeros); off[] holds
// each lane's byte offsets, which carry the row stride and the LDS swizzle.
// Whether load u is a K or a V load: when NW divides KL it is a K load exactly when
// u < KL / NW (wave < NW), which STATIC_KV fixes at compile time (1.3 % faster on the dense
// forward); else the wave tests wave + NW u < KL. Both issue the same loads in the same
// order; the paged loader keeps the test (below).
template <typename C, bool STATIC_KV = true>
__device__ __forceinline__ void issue_kv_at(const char *kt, const char *vt,
                                            const unsigned (&off)[C::LPW], int rest, char *kdst,
                                            char *vdst, int wave)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kt), (short)0, rest, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vt), (short)0, rest, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int i = wave + C::NW * u;
        if (STATIC_KV && C::KL % C::NW == 0 ? u < C::KL / C::NW : i < C::KL)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(kdst + i * 1024), 16, off[u],
                                                     0, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(vdst + (i - C::KL) * 1024),
                                                     16, off[u], 0, 0, 0);
    }
#endif
}

// Tiles of contiguous [N, D] rows (K and V of one batch-head): tile starting at key kv0.
template <typename C>
__device__ __forceinline__ void issue_kv(const char *kbh, const char *vbh,
                                         const unsigned (&off)[C::LPW], int kv0, int Nkv,
                                         char *kdst, char *vdst, int wave)
{
    kv0 = __builtin_amdgcn_readfirstlane(kv0);
    const int rest = (int)((unsigned)(Nkv - kv0) * C::ROWB);
    issue_kv_at<C>(kbh + (size_t)kv0 * C::ROWB, vbh + (size_t)kv0 * C::ROWB, off, rest, kdst,
                   vdst, wave);
}

// A paged K/V cache: pages of kPageTokens tokens laid out [num_pages, kPageTokens, H, D];
// logical token j of sequence s is slot j % kPageTokens of page table[s * max_pages +
// j / kPageTokens]. Query chunks are [S, Qmax, H, D] (row i of sequence s at (s Qmax + i) H + h),
// LSE [S, Qmax, H].
constexpr int kPageTokens = 256;

// Where a forward launch finds its keys and values.
//  kKvDense:   K, V [B, H, Nkv, d] contiguous.
//  kKvPaged:   a paged cache (fields table .. H); query chunks token-major, see above.
//  kKvTwoPart: keys [0, n1) from K, V [B, H, n1, d] and keys [n1, Nkv) from k2, v2
//              [B, H, Nkv - n1, d]; n1 is a multiple of the 32-key tile, so no tile spans both.
constexpr int kKvDense = 0, kKvPaged = 1, kKvTwoPart = 2;
struct KvLayout {
    const int32_t *table, *seq_lens, *q_lens;
    int max_pages, num_pages, Qmax, H;
    const uint16_t *k2, *v2;
    int n1;
};

// The K and V tiles of keys [kv0, kv0 + 32) of a paged sequence; page_at: byte offset of the
// head's first row in the tile's page (a tile never crosses a page). The K-or-V choice of each
// load stays a run-time test here: with it fixed at compile time the paged kernel ran as fast
// but read 6-8 % more from HBM (more K/V tiles fetched twice by the query tiles of a (sequence,
// head) pair, whose rows share L2 sets: a head's rows sit 8 KB apart in every 2 MB page),
// on every input measured.
template <typename C>
__device__ __forceinline__ void issue_kv_paged(const char *kpool, const char *vpool,
                                               size_t page_at, int H,
                                               const unsigned (&off)[C::LPW], unsigned kv0,
                                               int Nkv, char *kdst, char *vdst, int wave)
{
    const size_t at = page_at + (kv0 % kPageTokens) * (unsigned)(H * C::ROWB);
    const int rows = min(Nkv - (int)kv0, C::BN);
    const int rest = rows * H * C::ROWB;
    issue_kv_at<C, false>(kpool + at, vpool + at, off, rest, kdst, vdst, wave);
}

// Element mask of a 32-key score tile starting at kv0, for query row ip (lane half g):
// hidden scores become -inf (unscaled; the scale is applied with the exponent).
template <int MASK>
__device__ __forceinline__ void mask_tile(f32x16 &s, int kv0, int ip, int Nkv, int W, int G,
                                          int g)
{
    const int base = kv0 + 4 * g;
    const int hiR = (MASK == 0 || MASK == 4 ? Nkv - 1
                     : MASK == 3            ? min(ip + W, Nkv - 1)
                                            : min(ip, Nkv - 1)) -
                    base;
    const int loR = (MASK == 2 ? ip - W + 1 : MASK == 3 ? ip - W : INT_MIN / 2) - base;
    const int gR = (MASK == 2 || MASK == 4 ? G : 0) - base;
    const int cR = ip - base;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + (e & 3);
        bool vis = r <= hiR;
        if (MASK == 2) vis = vis && (r >= loR || r < gR);
        if (MASK == 3) vis = vis && r >= loR;
        if (MASK == 4) vis = vis && (r <= cR || r < gR);
        s[e] = vis ? s[e] : -INFINITY;
    }
}

__device__ __forceinline__ float max16(const f32x16 &v)
{
    // a tree of three-input maxima: 5 + 2 + 1 instructions
    const float r0 = vmax(vmax(v[0], v[1]), v[2]), r1 = vmax(vmax(v[3], v[4]), v[5]);
    const float r2 = vmax(vmax(v[6], v[7]), v[8]), r3 = vmax(vmax(v[9], v[10]), v[11]);
    const float r4 = vmax(vmax(v[12], v[13]), v[14]);
    return vmax(vmax(vmax(r0, r1), r2), vmax(vmax(r3, r4), v[15]));
}

}  // namespace
}  // namespace teaf
