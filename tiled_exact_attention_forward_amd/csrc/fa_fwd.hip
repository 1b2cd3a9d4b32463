// fa_fwd.hip -- tiled exact attention forward pass for gfx950 (MI355X, CDNA4).
//
// Method (ops-transformer article on gitcode.csdn.net, section 二.1 "FlashAttention算子";
// zwxr.cn article, section 3.1): a workgroup owns one tile of query rows, keeps them on
// chip, and walks the key/value tiles that its mask leaves visible. Per tile it forms the
// score block on the matrix cores, updates a running row maximum m and running sum l
// (online softmax), rescales the output accumulator by exp(m_old - m_new) and adds P V.
// After the last tile the accumulator is divided by l once. The N x N scores never leave
// registers. Scores, m, l and the accumulator are fp32 (the pages keep the softmax
// denominator in fp32); P is rounded to the input type for the P V product.
//
// gfx950 mapping (not the pages' Ascend tiling, which was sized for the 910's buffers):
//  * 256 threads = 4 wave64s, 128 query rows per workgroup, 32 rows per wave, two
//    workgroups per CU; key/value tiles of 32 rows.
//  * K and V tiles go straight from HBM into a 4-slot LDS ring (buffer_load ... lds), two
//    tiles ahead of their first use; a workgroup barrier per tile waits only for LDS traffic
//    and for the one tile it publishes.
//  * The score block is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,
//    f16}: lane (g, i) then holds 16 keys of query row i per 32-key tile, so the row max
//    and row sum are in-lane reductions plus one cross-half register swap, and the fp32
//    accumulator converts in place into the B operand (P^T) of O^T = V^T P^T.
//  * Software pipeline per wave: the matrix cores compute the scores of tile t+1 while the
//    vector unit exponentiates tile t, then accumulate P(t) V(t) while the vector unit sums
//    P(t) and takes the maximum of tile t+1; scheduling barriers fix that order.
//  * V stays row-major in LDS; the V^T operand is read with ds_read_b64_tr_b16, whose
//    16-lane transpose hands each lane four consecutive keys of one column.
//  * exp(x) is evaluated as 2^(x log2 e) with v_exp_f32; the log2 e factor is folded into
//    the score scale, which enters through the FMA that subtracts the row maximum.
//  * Tiles that a mask hides from every row are never loaded; tiles every row sees
//    completely skip the element mask, which only edge tiles evaluate.
//  * Workgroup ids are remapped so the query tiles of one (batch, head) run on one XCD and
//    share its L2 copy of K and V; the query tiles with the most visible keys go first.
//
// fp32 inputs use v_mfma_f32_32x32x2f32 (true fp32 products) in a simpler single-buffered
// kernel with 32-key tiles.
#include <limits.h>
#include <math.h>

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

// The running maximum is only moved (and O, l rescaled) when a row's new maximum exceeds
// the one in use by more than this many powers of two; until then probabilities are taken
// relative to the stale maximum and stay below 2^8, which fp32 sums and 16-bit P hold
// exactly as well. The result is the same softmax: numerator and denominator share the
// reference value, and the final division removes it.
constexpr float kRescaleSlack = 8.0f;

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
template <typename C>
__device__ __forceinline__ void issue_kv(const char *kbh, const char *vbh,
                                         const unsigned (&off)[C::LPW], int kv0, int Nkv,
                                         char *kdst, char *vdst, int wave)
{
#if defined(__HIP_DEVICE_COMPILE__)
    kv0 = __builtin_amdgcn_readfirstlane(kv0);
    const int rest = (int)((unsigned)(Nkv - kv0) * C::ROWB);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(kbh + (size_t)kv0 * C::ROWB), (short)0, rest, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(vbh + (size_t)kv0 * C::ROWB), (short)0, rest, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int i = wave + C::NW * u;
        if (i < C::KL)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(kdst + i * 1024), 16, off[u],
                                                     0, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(vdst + (i - C::KL) * 1024),
                                                     16, off[u], 0, 0, 0);
    }
#endif
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
    const float a = vmax(vmax(vmax(v[0], v[1]), vmax(v[2], v[3])),
                         vmax(vmax(v[4], v[5]), vmax(v[6], v[7])));
    const float b = vmax(vmax(vmax(v[8], v[9]), vmax(v[10], v[11])),
                         vmax(vmax(v[12], v[13]), vmax(v[14], v[15])));
    return vmax(a, b);
}

// One pipeline step for tile t. sc: raw scores of tile t (masked if needed), mt its
// scaled row maximum. NEXT: there is a tile t+1 (K in LDS at kn); mask_next: it needs the
// element mask (wave-uniform). vc: V of tile t in LDS.
template <typename T, typename C, int MASK, bool NEXT>
__device__ __forceinline__ void sp_step(const char *__restrict__ kn, const char *__restrict__ vc,
                                        const int (&kofs)[C::NKK], const int (&vofs)[C::NDB],
                                        const s16x8 (&qf)[C::NKK], f32x16 (&oacc)[C::NDB],
                                        f32x16 &sc, f32x16 &sn, float &m, float &l, float &mt,
                                        float c, bool mask_next, int kvn, int ip, int Nkv, int W,
                                        int G, int g)
{
    using Op = Ops16<T>;
    constexpr int NKK = C::NKK, NDB = C::NDB, KPF = C::KPF, VPF = C::VPF;
    constexpr int EPK = 16 / NKK;   // probabilities formed per score instruction
    constexpr int NF = 2 * NDB;     // P V matrix instructions

    // K fragment reads for the first matrix instructions go out before the rescale test.
    s16x8 kf[NKK];
    if (NEXT) {
#pragma unroll
        for (int f = 0; f < KPF; ++f) kf[f] = *(const s16x8 *)(kn + kofs[f]);
    }
    if (!__all(mt <= m + kRescaleSlack)) {
        const float mn = fmaxf(m, mt);
        const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
        m = mn;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    const float nmu = (m == -INFINITY) ? 0.f : -m;
    __builtin_amdgcn_sched_barrier(0);

    // Phase A: S(t+1) = K(t+1) Q^T, P(t) = 2^(c S(t) - m).
    s16x4 vlo[NF], vhi[NF];
    auto vread = [&](int f) {
        const int kc = f / NDB, db = f % NDB;
        const char *p0 = vc + vofs[db] + kc * 16 * C::ROWB;
        vlo[f] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
        vhi[f] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 8 * C::ROWB));
    };
    s16x8 pf[2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (NEXT) {
            if (kk + KPF < NKK) kf[kk + KPF] = *(const s16x8 *)(kn + kofs[kk + KPF]);
            sn = Op::mma(kf[kk], qf[kk], kk == 0 ? f32x16{} : sn);
        }
        if (kk >= NKK - VPF) vread(kk - (NKK - VPF));
#pragma unroll
        for (int e = kk * EPK; e < (kk + 1) * EPK; ++e)
            sc[e] = fast_exp2(__builtin_fmaf(sc[e], c, nmu));
        if (((kk + 1) * EPK) % 8 == 0) {
            const int o = (kk + 1) * EPK - 8;
            pf[o / 8] = Op::pack8(sc[o], sc[o + 1], sc[o + 2], sc[o + 3], sc[o + 4], sc[o + 5],
                                  sc[o + 6], sc[o + 7]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Phase B: O^T += V^T P^T(t); l += row sums of P(t); mask and maximum of S(t+1).
    float ps[4];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int kc = f / NDB, db = f % NDB;
        if (f + VPF < NF) vread(f + VPF);
        const s16x8 a = __builtin_shufflevector(vlo[f], vhi[f], 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = Op::mma(a, pf[kc], oacc[db]);
        // vector work spread over the matrix instructions
        if (NF == 8) {
            if (f < 4) ps[f] = (sc[4 * f] + sc[4 * f + 1]) + (sc[4 * f + 2] + sc[4 * f + 3]);
            if (f == 4) l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
            if (NEXT && f == 4 && mask_next) mask_tile<MASK>(sn, kvn, ip, Nkv, W, G, g);
            if (NEXT && f == 6) mt = half_swap_max(max16(sn)) * c;
        } else {
            if (f == 0) {
                ps[0] = (sc[0] + sc[1]) + (sc[2] + sc[3]);
                ps[1] = (sc[4] + sc[5]) + (sc[6] + sc[7]);
            }
            if (f == 1) {
                ps[2] = (sc[8] + sc[9]) + (sc[10] + sc[11]);
                ps[3] = (sc[12] + sc[13]) + (sc[14] + sc[15]);
                l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
            }
            if (NEXT && f == 2 && mask_next) mask_tile<MASK>(sn, kvn, ip, Nkv, W, G, g);
            if (NEXT && f == 3) mt = half_swap_max(max16(sn)) * c;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <typename T, int D, int MASK, int NS, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int Nq,
    int Nkv, float c, int W, int G, int nqt, const uint8_t *__restrict__ layout, int H)
{
    using C = CfgSP<D, NS, NW>;
    using Op = Ops16<T>;
    constexpr int BM = C::BM, BN = C::BN, LPW = C::LPW;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - L % nqt) * BM;  // most-loaded query tiles first
    const int delta = Nkv - Nq;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;

    // Q^T fragments (B operand): lane (g, i) holds Q[row i][16kk + 8g .. +7]. The loads go
    // out back to back ahead of the first K/V tiles (padding rows read the last row) and are
    // finished after the wait for those tiles, so no wait sits between them. A negative
    // scale is moved into Q by flipping sign bits (exact). c is kept at least the smallest
    // normal float so that a hidden score (-inf) times c stays -inf; for |scale| below
    // that every visible weight is 2^0 either way.
    const int row = q0 + wave * 32 + li;
    const int ip = row + delta;
    const short qsign = c < 0.f ? (short)0x8000 : (short)0;
    c = fmaxf(fabsf(c), 1.17549435e-38f);
    s16x8 qf[C::NKK];
    {
        const uint16_t *qr = Q + qbase + (size_t)min(row, Nq - 1) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) qf[kk] = *(const s16x8 *)(qr + 16 * kk);
    }

    char *const lds = (char *)smem;
    // Range schedule (masks 0-4), or for the block-sparse mask a list of the visible key
    // blocks of this query block, built in LDS after the K/V ring.
    const TileSchedule sch = make_schedule<MASK == kBlockSparse ? 0 : MASK, BM, BN>(
        q0, Nq, Nkv, W, G);
    int ntl = sch.total, nint = sch.interior;
    const uint16_t *blist = (const uint16_t *)(lds + C::LDS_BYTES + 16);
    const int tail_kv0 = ((Nkv + BN - 1) / BN - 1) * BN;  // first key of the last key tile
    if constexpr (MASK == kBlockSparse) {
        static_assert(BM == kSparseBlock && kSparseBlock % BN == 0, "one query block per tile");
        constexpr int TPB = kSparseBlock / BN, CH = kMaxKeyBlocks / (64 * NW);
        const int nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        const uint8_t *lrow = layout + ((size_t)(bh % H) * nqt + q0 / kSparseBlock) * nkb;
        int *wcnt = (int *)(lds + C::LDS_BYTES);
        uint16_t *bl = (uint16_t *)(lds + C::LDS_BYTES + 16);
        bool f[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {  // all layout loads first, one wait
            const int b = u * 64 * NW + tid;
            f[u] = b < nkb && lrow[b] != 0;
        }
        int n = 0;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            if (u * 64 * NW >= nkb) break;
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
                bl[n + before + __popcll(mk & ((1ull << lane) - 1))] =
                    (uint16_t)(u * 64 * NW + tid);
            n += total;
            __syncthreads();
        }
        // stream position p holds tile TPB * blist[p / TPB] + p % TPB; only the final key
        // block can have fewer tiles, and it comes last; only the key-tail tile is masked
        if (n == 0) {
            ntl = nint = 0;
        } else {
            const int lastb = __builtin_amdgcn_readfirstlane((int)bl[n - 1]);
            const int all = (Nkv + BN - 1) / BN;
            ntl = TPB * (n - 1) + (lastb == nkb - 1 ? all - TPB * lastb : TPB);
            nint = ntl - (lastb == nkb - 1 && Nkv % BN != 0 ? 1 : 0);
        }
    }
    auto bs_tile = [&](int p) {
        constexpr int TPB = kSparseBlock / BN;
        return __builtin_amdgcn_readfirstlane((int)blist[p / TPB] * TPB + p % TPB);
    };

    float m = -INFINITY, l = 0.f;
    f32x16 oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};

    const char *kbh = (const char *)(K + kvbase);
    const char *vbh = (const char *)(V + kvbase);
    // Load u of this wave fills rows r of the K (or V) tile; lane l lands in physical chunk
    // l % CHUNKS of row r = first + l / CHUNKS, so it fetches the logical chunk the swizzle
    // stores there. Offsets are relative to the tile's first key.
    unsigned off[C::LPW];
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int i = wave + NW * u;
        const int r = (i % C::KL) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        const int pc = lane % C::CHUNKS;
        off[u] = r * C::ROWB + 16 * (i < C::KL ? k_swz<D>(r, pc) : v_swz<D>(r, pc));
    }
    int kofs[C::NKK], vofs[C::NDB];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * k_swz<D>(li, 2 * kk + g);
    {
        const int trow = 4 * g + ((lane & 15) >> 2);
        const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
            vofs[db] = trow * C::ROWB + 16 * v_swz<D>(trow, 4 * db + tchunk) + 8 * (lane & 1);
    }

    auto kslot = [&](int t) { return lds + (t % NS) * C::TILEB; };
    auto vslot = [&](int t) { return lds + C::VREG + (t % NS) * C::TILEB; };

    // Prologue: tiles 0 .. NS-2 in flight; wait for tiles 0 and 1.
    TileSchedule::Cursor ld = sch.begin();
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
        if (j < ntl) {
            const int tl = MASK == kBlockSparse ? bs_tile(j) : ld.t;
            issue_kv<C>(kbh, vbh, off, tl * BN, Nkv, kslot(j), vslot(j), wave);
            ld = sch.next(ld);
        }
    }
    wait_tiles<LPW, NS - 3>(min(NS - 1, ntl) - 2);
    ring_barrier();
    {
        const short keep = row < Nq ? (short)-1 : (short)0;
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) qf[kk] = (qf[kk] ^ qsign) & keep;
    }

    f32x16 sa, sb;
    float mt = -INFINITY;
    TileSchedule::Cursor nx = sch.begin();
    if (ntl > 0) {
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
            sa = Op::mma(*(const s16x8 *)(kslot(0) + kofs[kk]), qf[kk],
                         kk == 0 ? f32x16{} : sa);
        if (nint == 0)
            mask_tile<MASK == kBlockSparse ? 0 : MASK>(
                sa, MASK == kBlockSparse ? tail_kv0 : nx.t * BN, ip, Nkv, W, G, g);
        mt = half_swap_max(max16(sa)) * c;
        nx = sch.next(nx);
    }

    // Step t: load tile t+NS-1, finish tile t, start tile t+1; then make tile t+2 resident.
    auto step_end = [&](int t) {
        wait_tiles<LPW, NS - 3>(min(t + NS - 1, ntl - 1) - (t + 2));
        ring_barrier();
    };
    auto load_ahead = [&](int t) {
        if (t + NS - 1 < ntl) {
            const int tl = MASK == kBlockSparse ? bs_tile(t + NS - 1) : ld.t;
            issue_kv<C>(kbh, vbh, off, tl * BN, Nkv, kslot(t + NS - 1), vslot(t + NS - 1),
                        wave);
            ld = sch.next(ld);
        }
    };
    // Two steps per iteration so that sa and sb swap roles without register copies. Every
    // step in the loop has a tile t+1; the last step is peeled.
    auto step = [&](int t, f32x16 &cur, f32x16 &nxt) {
        load_ahead(t);
        sp_step<T, C, MASK == kBlockSparse ? 0 : MASK, true>(
            kslot(t + 1), vslot(t), kofs, vofs, qf, oacc, cur, nxt, m, l, mt, c, t + 1 >= nint,
            MASK == kBlockSparse ? tail_kv0 : nx.t * BN, ip, Nkv, W, G, g);
        nx = sch.next(nx);
        step_end(t);
    };
    auto last = [&](int t, f32x16 &cur, f32x16 &nxt) {
        sp_step<T, C, MASK == kBlockSparse ? 0 : MASK, false>(
            nullptr, vslot(t), kofs, vofs, qf, oacc, cur, nxt, m, l, mt, c, false, 0, ip, Nkv, W,
            G, g);
    };
    if (ntl > 0) {
        int t = 0;
        for (; t + 2 < ntl; t += 2) {
            step(t, sa, sb);
            step(t + 1, sb, sa);
        }
        if (t + 1 < ntl) {
            step(t, sa, sb);
            last(t + 1, sb, sa);
        } else {
            last(t, sa, sb);
        }
    }

    // Epilogue: both lane halves hold partial sums of the same row (same reference max).
    const float lt = half_swap_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row < Nq) {
        uint16_t *orow = O + qbase + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const s16x4 v4 = Op::pack4(oacc[db][4 * blk + 0] * inv, oacc[db][4 * blk + 1] * inv,
                                           oacc[db][4 * blk + 2] * inv, oacc[db][4 * blk + 3] * inv);
                *(s16x4 *)(orow + db * 32 + 8 * blk + 4 * g) = v4;
            }
        }
        if (g == 0)
            LSE[(size_t)bh * Nq + row] =
                lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
}

// ------------------------------------------------------------------ fp32 kernel

template <int D, int MASK>
__global__ __launch_bounds__(256) void fwd32_kernel(const float *__restrict__ Q,
                                                    const float *__restrict__ K,
                                                    const float *__restrict__ V,
                                                    float *__restrict__ O, float *__restrict__ LSE,
                                                    int Nq, int Nkv, float c, int W, int G, int nqt,
                                                    const uint8_t *__restrict__ layout, int H)
{
    constexpr int BM = 128, BN = 32, NT = 256, KP = D + 1;
    constexpr int NKK = D / 2, NDB = D / 32, RC = D / 4, CPT = BN * RC / NT;
    __shared__ float ks[BN * KP];
    __shared__ __attribute__((aligned(16))) float vs[BN * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - L % nqt) * BM;
    const int delta = Nkv - Nq;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;
    const int wrow0 = q0 + wave * 32, row = wrow0 + li, ip = row + delta;

    // Q^T fragments for the 32x32x2 MFMA: lane (g, i) holds Q[row i][2kk + g].
    float qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = row < Nq ? Q[qbase + (size_t)row * D + 2 * kk + g] : 0.f;

    const TileRanges tr = visible_tiles<MASK, BM, BN>(q0, Nq, Nkv, W, G);
    const int na = tr.a1 - tr.a0, ntiles = na + (tr.b1 - tr.b0);
    float m = -INFINITY, l = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;

    const uint8_t *lrow = nullptr;
    if (MASK == kBlockSparse) {
        const int nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        lrow = layout + ((size_t)(bh % H) * nqt + q0 / kSparseBlock) * nkb;
    }
    for (int n = 0; n < ntiles; ++n) {
        const int tile = n < na ? tr.a0 + n : tr.b0 + (n - na);
        const int kv0 = tile * BN;
        if (MASK == kBlockSparse && lrow[kv0 / kSparseBlock] == 0) continue;  // whole workgroup
        __syncthreads();  // previous tile's readers are done
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int id = tid + u * NT, r = id / RC, cc = id % RC, key = kv0 + r;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (key < Nkv) {
                kv = *(const f32x4 *)(K + kvbase + (size_t)key * D + 4 * cc);
                vv = *(const f32x4 *)(V + kvbase + (size_t)key * D + 4 * cc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ks[r * KP + 4 * cc + e] = kv[e];
            *(f32x4 *)(vs + r * D + 4 * cc) = vv;
        }
        __syncthreads();

        bool skip = wrow0 >= Nq;
        bool need_mask = kv0 + BN > Nkv || MASK == 3 || MASK == 4;
        if (MASK == 1 || MASK == 2) {
            const int ip0 = wrow0 + delta, ip1 = wrow0 + 31 + delta;
            if (kv0 > ip1) skip = true;
            if (kv0 + BN - 1 > ip0) need_mask = true;
            if (MASK == 2) {
                if (kv0 + BN - 1 < ip0 - W + 1 && kv0 >= G) skip = true;
                if (!(ip1 - kv0 < W) && !(kv0 + BN - 1 < G)) need_mask = true;
            }
        }
        if (skip) continue;

        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[li * KP + 2 * kk + g], qf[kk], sacc, 0, 0, 0);
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float t = sacc[e] * c;
            if (need_mask) {
                const int key = kv0 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (key >= Nkv || !key_visible<MASK>(ip, key, W, G)) t = -INFINITY;
            }
            sacc[e] = t;
            mt = fmaxf(mt, t);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        m = mn;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(sacc[e] - mu);
            sacc[e] = p;
            ps += p;
        }
        l = l * alpha + ps;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        // O^T += V^T P^T, one key per lane half per step: key 8blk + 4g + r.
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + db * 32 + li], sacc[e],
                                                                oacc[db], 0, 0, 0);
        }
    }

    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row < Nq) {
        float *orow = O + qbase + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                f32x4 v4 = {oacc[db][4 * blk] * inv, oacc[db][4 * blk + 1] * inv,
                            oacc[db][4 * blk + 2] * inv, oacc[db][4 * blk + 3] * inv};
                *(f32x4 *)(orow + db * 32 + 8 * blk + 4 * g) = v4;
            }
        if (g == 0)
            LSE[(size_t)bh * Nq + row] =
                lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
}

// 4 waves (128 query rows) per workgroup, two workgroups per CU, a 4-slot K/V ring.
constexpr int kStages = 4, kWaves = 4;

template <typename T, int D, int MASK>
hipError_t launch16(const FwdArgs &a, hipStream_t s)
{
    using C = CfgSP<D, kStages, kWaves>;
    const int nqt = (a.Nq + C::BM - 1) / C::BM;
    const long nblk = (long)nqt * a.B * a.H;
    auto kern = fwd16_kernel<T, D, MASK, kStages, kWaves>;
    // block sparse: wave counts and the key-block list (2 bytes a block) after the ring
    const int lds = MASK == kBlockSparse ? C::LDS_BYTES + 16 + 2 * kMaxKeyBlocks : C::LDS_BYTES;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NT), lds, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (uint16_t *)a.o, a.lse, a.Nq, a.Nkv, a.scale * kLog2e, a.window,
                       a.n_global, nqt, a.layout, a.H);
    return hipGetLastError();
}

template <int D, int MASK>
hipError_t launch32(const FwdArgs &a, hipStream_t s)
{
    const int nqt = (a.Nq + 127) / 128;
    const long nblk = (long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd32_kernel<D, MASK>), dim3((unsigned)nblk), dim3(256), 0, s,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, (float *)a.o,
                       a.lse, a.Nq, a.Nkv, a.scale * kLog2e, a.window, a.n_global, nqt,
                       a.layout, a.H);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch16_mask(const FwdArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch16<T, D, 0>(a, s);
    case 1: return launch16<T, D, 1>(a, s);
    case 2: return launch16<T, D, 2>(a, s);
    case 3: return launch16<T, D, 3>(a, s);
    case 4: return launch16<T, D, 4>(a, s);
    default: return launch16<T, D, kBlockSparse>(a, s);
    }
}

template <int D>
hipError_t launch32_mask(const FwdArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch32<D, 0>(a, s);
    case 1: return launch32<D, 1>(a, s);
    case 2: return launch32<D, 2>(a, s);
    case 3: return launch32<D, 3>(a, s);
    case 4: return launch32<D, 4>(a, s);
    default: return launch32<D, kBlockSparse>(a, s);
    }
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t s)
{
    (void)hipGetLastError();  // start from a clean error state
    if (a.dtype == 0) return a.d == 64 ? launch32_mask<64>(a, s) : launch32_mask<128>(a, s);
    if (a.dtype == 1)
        return a.d == 64 ? launch16_mask<_Float16, 64>(a, s) : launch16_mask<_Float16, 128>(a, s);
    return a.d == 64 ? launch16_mask<__bf16, 64>(a, s) : launch16_mask<__bf16, 128>(a, s);
}

}  // namespace teaf
