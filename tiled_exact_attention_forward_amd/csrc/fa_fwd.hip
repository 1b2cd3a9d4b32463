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
#include <algorithm>

#include "fa_device.h"

namespace teaf {
namespace {

// Online softmax without a per-tile row maximum. The probabilities of tile t are formed as
// 2^(c s - m) against the reference m in use, and the tile's row sums (formed anyway for l)
// are checked before the probabilities are used: while every partial sum of 16 probabilities
// stays at most the bound, every probability is below it, so fp32 sums of up to 2^31 keys,
// P in the input type and the fp32 accumulator all stay finite and keep their relative
// precision, and the result is the same softmax (numerator and denominator share the
// reference, the final division removes it). The bound is 2^64 for bf16 (fp32's exponent
// range) and 2^15 for fp16, whose largest finite value is 65504. A sum above the bound, an
// infinity or a NaN, or any visible key for a row that had none (its reference is still
// -inf; there the bound is 0), sends the wave to the rare exact path: the tile's scores are
// formed again, the reference becomes the true running maximum and the accumulator and sum
// are rescaled. This takes no maximum over the scores of ordinary tiles: the first tile of a
// query tile sets the reference.
template <typename T>
constexpr float sum_bound()
{
    return __is_same(T, _Float16) ? 32768.f : 18446744073709551616.f;
}

// One pipeline step for tile t. sc: raw scores of tile t (masked if needed). m: scaled
// reference maximum, nmu = -m (0 while m is -inf), bnd: the row-sum bound (0 while m is
// -inf); all three change only on the rare path. NEXT: there is a tile t+1 (K in LDS at kn);
// mask_next: it needs the element mask (wave-uniform), kvn its first key. kc: K of tile t
// (for the rare path), mask_cur and kvc: its mask and first key. vslot_ofs: where V of tile t
// sits in the V ring (bytes from the ring's first slot); vptr: this lane's V^T read addresses
// in the first slot.
template <typename T, typename C, int MASK, bool NEXT>
__device__ __forceinline__ void sp_step(const char *__restrict__ kn, const char *__restrict__ kc,
                                        unsigned vslot_ofs, const int (&kofs)[C::NKK],
                                        const lds_char *const (&vptr)[C::NDB],
                                        const s16x8 (&qf)[C::NKK], f32x16 (&oacc)[C::NDB],
                                        f32x16 &sc, f32x16 &sn, float &m, float &nmu, float &bnd,
                                        float &l, float c, bool mask_cur, int kvc,
                                        bool mask_next, int kvn, int ip, int Nkv, int W, int G,
                                        int g)
{
    using Op = Ops16<T>;
    constexpr int NKK = C::NKK, NDB = C::NDB, KPF = C::KPF, VPF = C::VPF;
    constexpr int EPK = 16 / NKK;   // probabilities formed per score instruction
    constexpr int NF = 2 * NDB;     // P V matrix instructions

    s16x8 kf[NKK];
    if (NEXT) {
#pragma unroll
        for (int f = 0; f < KPF; ++f) kf[f] = *(const s16x8 *)(kn + kofs[f]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // The wave runs phase A at raised priority: of the two waves sharing a SIMD, the one
    // issuing the score MFMAs and exponentials goes first (about 1 % faster, measured).
    __builtin_amdgcn_s_setprio(1);
    // Phase A: S(t+1) = K(t+1) Q^T; P(t) = 2^(c S(t) - m) and its row sums.
    s16x4 vlo[NF], vhi[NF];
    // V^T reads: per-lane LDS addresses made once per workgroup; the slot (a constant in
    // the unrolled loop) and the chunk enter as immediate offsets.
    auto vread = [&](int f) {
        const int kcn = f / NDB, db = f % NDB;
        const lds_char *p0 = vptr[db] + vslot_ofs + kcn * 16 * C::ROWB;
        vlo[f] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
        vhi[f] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 8 * C::ROWB));
    };
    s16x8 pf[2];
    float ps[4];
    auto prob = [&](int e) { sc[e] = fast_exp2(__builtin_fmaf(sc[e], c, nmu)); };
    auto pack = [&](int o) {
        pf[o / 8] = Op::pack8(sc[o], sc[o + 1], sc[o + 2], sc[o + 3], sc[o + 4], sc[o + 5],
                              sc[o + 6], sc[o + 7]);
    };
    auto psum = [&](int q) {
        ps[q] = (sc[4 * q] + sc[4 * q + 1]) + (sc[4 * q + 2] + sc[4 * q + 3]);
    };
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        // The first group's exponentials go ahead of the first score instruction, covering
        // the latency of the K fragment reads that follow the step's barrier.
        if (kk == 0) {
#pragma unroll
            for (int e = 0; e < EPK; ++e) prob(e);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (NEXT) {
            if (kk + KPF < NKK) kf[kk + KPF] = *(const s16x8 *)(kn + kofs[kk + KPF]);
            sn = Op::mma(kf[kk], qf[kk], kk == 0 ? f32x16{} : sn);
        }
        if (kk >= NKK - VPF) vread(kk - (NKK - VPF));
#pragma unroll
        for (int e = kk * EPK; e < (kk + 1) * EPK; ++e)
            if (kk > 0) prob(e);
        const int done = (kk + 1) * EPK;  // probabilities formed so far
        if (done % 4 == 0) psum(done / 4 - 1);
        if (done % 8 == 0) pack(done - 8);
        __builtin_amdgcn_sched_barrier(0);
    }
    float pt = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    if (!__all(pt <= bnd)) {
        // Rare path: the tile's scores again (K(t) is still in its slot), its true maximum as
        // the new reference, the accumulator and sum rescaled, the tile's probabilities anew.
        f32x16 s;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            s = Op::mma(*(const s16x8 *)(kc + kofs[kk]), qf[kk], kk == 0 ? f32x16{} : s);
        if (mask_cur) mask_tile<MASK>(s, kvc, ip, Nkv, W, G, g);
        const float mt = half_swap_max(max16(s)) * c;
        const float mn = fmaxf(m, mt);
        const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
        m = mn;
        nmu = mn == -INFINITY ? 0.f : -mn;
        bnd = mn == -INFINITY ? 0.f : sum_bound<T>();
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        sc = s;
#pragma unroll
        for (int e = 0; e < 16; ++e) prob(e);
#pragma unroll
        for (int q = 0; q < 4; ++q) psum(q);
        pack(0);
        pack(8);
        pt = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
    l += pt;

    __builtin_amdgcn_s_setprio(0);
    // Phase B: O^T += V^T P^T(t); the element mask of S(t+1) when it needs one.
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int kcn = f / NDB, db = f % NDB;
        if (f + VPF < NF) vread(f + VPF);
        const s16x8 a = __builtin_shufflevector(vlo[f], vhi[f], 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = Op::mma(a, pf[kcn], oacc[db]);
        if (NEXT && f == NF / 2 && mask_next) mask_tile<MASK>(sn, kvn, ip, Nkv, W, G, g);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// KVL (kKvDense, kKvPaged, kKvTwoPart) says where the keys are, see KvLayout. Paged: the
// query rows are a chunk of the newest tokens of sequence bh / H (head bh % H) and K/V come
// from the page pool described by pg; Nq and Nkv are then that sequence's chunk and cache
// lengths, read from pg (the arguments are ignored). Two parts: key tiles below pg.n1 come
// from K and V, the rest from pg.k2 and pg.v2.
// Launch bound: NW waves per workgroup, at least two waves per SIMD (256 registers each).
template <typename T, int D, int MASK, int NS, int NW, int KVL>
__global__ __launch_bounds__(64 * NW, 2) void fwd16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int Nq,
    int Nkv, float c, int W, int G, int nqt, const uint8_t *__restrict__ layout, int H,
    const KvLayout pg)
{
    constexpr bool PAGED = KVL == kKvPaged;
    using C = CfgSP<D, NS, NW>;
    using Op = Ops16<T>;
    constexpr int BM = C::BM, BN = C::BN, LPW = C::LPW;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    int bh = L / nqt;
    int q0 = (nqt - 1 - L % nqt) * BM;  // most-loaded query tiles first
    // Row strides (elements) of Q and O, and where this workgroup's rows and LSE entries
    // start. Lengths in a paged cache are clamped to what the table and the chunk can hold.
    int rs = D;
    size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D, lbase = (size_t)bh * Nq;
    if (KVL == kKvTwoPart) kvbase = (size_t)bh * pg.n1 * D;
    int lstride = 1, seq = 0, head = 0;
    if constexpr (PAGED) {
        // (sequence, head) pairs are spread so that every XCD receives H/8 heads of every
        // sequence (a sequence per XCD left the XCD with the longest history last), and
        // within an XCD's share the pairs go sequence by sequence with adjacent heads, so
        // the pairs running side by side read neighbouring heads of the same pages (the
        // same head of different sequences sits at the same offset in pages 2 MB apart and
        // competes for the same L2 sets). The query tiles of a pair stay on one XCD and are
        // dispatched together, so they read each K/V tile while it is in that XCD's L2.
        const int nseq = (int)gridDim.x / (nqt * pg.H);
        if (pg.H % kXcds == 0) {
            const int hx = pg.H / kXcds, per = nseq * hx;  // heads per sequence per XCD
            const int x = bh / per, k = bh % per;
            seq = k / hx;
            // Up to 64 sequences go in order of decreasing work (chunk length times history,
            // ties by index), so the workgroups an XCD runs side by side have similar
            // lengths and finish together, and the query tiles of a pair start together.
            if (nseq <= 64) {
                const int sl = lane < nseq ? pg.seq_lens[lane] : 0;
                const int ql = lane < nseq ? pg.q_lens[lane] : 0;
                const long long wk = (long long)ql * (2LL * sl - ql);
                int rank = 0;
                for (int s2 = 0; s2 < nseq; ++s2) {
                    const long long w2 = __shfl(wk, s2);
                    rank += (w2 > wk || (w2 == wk && s2 < lane)) ? 1 : 0;
                }
                const unsigned long long hit = __ballot(lane < nseq && rank == seq);
                seq = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
            }
            head = hx * ((x + seq) % kXcds) + k % hx;
            // Within a pair the query tiles that hold rows come first (most loaded first),
            // the empty ones past the chunk's end last: an empty tile exits at once, and
            // ahead of its pair it let the next pair's tiles start before this pair's.
            const int qlen = min(min(__builtin_amdgcn_readfirstlane(pg.q_lens[seq]), pg.Qmax),
                                 __builtin_amdgcn_readfirstlane(pg.seq_lens[seq]));
            const int nt = (qlen + BM - 1) / BM, i = L % nqt;
            q0 = i < nt ? (nt - 1 - i) * BM : nqt * BM;
        } else {
            seq = bh % nseq;
            head = (bh / nseq + seq * max(1, pg.H / nseq)) % pg.H;
        }
        Nkv = min(__builtin_amdgcn_readfirstlane(pg.seq_lens[seq]), pg.max_pages * kPageTokens);
        Nq = min(min(__builtin_amdgcn_readfirstlane(pg.q_lens[seq]), pg.Qmax), Nkv);
        if (q0 >= Nq) return;  // the whole workgroup: this chunk is shorter
        rs = pg.H * D;
        qbase = ((size_t)seq * pg.Qmax * pg.H + head) * D;
        kvbase = 0;
        lbase = (size_t)seq * pg.Qmax * pg.H + head;
        lstride = pg.H;
    }
    const int delta = Nkv - Nq;

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
        const uint16_t *qr = Q + qbase + (size_t)min(row, Nq - 1) * rs + 8 * g;
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
        const int nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        const uint8_t *lrow = layout + ((size_t)(bh % H) * nqt + q0 / kSparseBlock) * nkb;
        key_block_list<NW, BN>(lds + C::LDS_BYTES, lrow, nkb, Nkv, tid, ntl, nint);
    }
    auto bs_tile = [&](int p) {
        constexpr int TPB = kSparseBlock / BN;
        return __builtin_amdgcn_readfirstlane((int)blist[p / TPB] * TPB + p % TPB);
    };

    float m = -INFINITY, nmu = 0.f, l = 0.f;
    f32x16 oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};

    const char *kbh = (const char *)(K + kvbase);
    const char *vbh = (const char *)(V + kvbase);
    auto kslot = [&](int t) { return lds + ((unsigned)t % NS) * C::TILEB; };
    auto vring_ofs = [&](int t) { return ((unsigned)t % NS) * C::TILEB; };
    auto vslot = [&](int t) { return lds + C::VREG + vring_ofs(t); };
    // Load u of this wave fills rows r of the K (or V) tile; lane l lands in physical chunk
    // l % CHUNKS of row r = first + l / CHUNKS, so it fetches the logical chunk the swizzle
    // stores there. Offsets are relative to the tile's first key.
    unsigned off[C::LPW];
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int i = wave + NW * u;
        const int r = (i % C::KL) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
        const int pc = lane % C::CHUNKS;
        off[u] = r * (PAGED ? pg.H * C::ROWB : C::ROWB) +
                 16 * (i < C::KL ? k_swz<D>(r, pc) : v_swz<D>(r, pc));
    }
    const int32_t *seq_table = PAGED ? pg.table + (size_t)seq * pg.max_pages : nullptr;
    // Paged: the ids of 64 consecutive pages of the sequence (from page pbase) sit one per
    // lane, so entering a page takes a register read, not a memory round trip; after 64
    // pages (16,384 keys) the walk loads the next 64 and waits for them there, which drains
    // the tiles in flight once. The page's offset in the pool is formed once per page.
    const int last_page = (Nkv - 1) / kPageTokens;
    unsigned pidx_cur = ~0u, pbase = 0;
    int ptab = 0;
    size_t page_at = 0;
    if constexpr (PAGED) ptab = lane <= last_page ? seq_table[lane] : 0;
    auto load_tile = [&](int tl, int slot) {
        if constexpr (PAGED) {
            const unsigned kv0 = __builtin_amdgcn_readfirstlane(tl * BN);
            const unsigned pidx = kv0 / kPageTokens;
            if (pidx != pidx_cur) {
                if (pidx - pbase >= 64u) {
                    pbase = pidx & ~63u;
                    ptab = (int)(pbase + lane) <= last_page ? seq_table[pbase + lane] : 0;
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                }
                const int pid = min(max(__builtin_amdgcn_readlane(ptab, pidx - pbase), 0),
                                    pg.num_pages - 1);
                pidx_cur = pidx;
                page_at = ((size_t)pid * kPageTokens * pg.H + head) * C::ROWB;
            }
            issue_kv_paged<C>(kbh, vbh, page_at, pg.H, off, kv0, Nkv, kslot(slot),
                              vslot(slot), wave);
        } else if constexpr (KVL == kKvTwoPart) {
            const int kv0 = __builtin_amdgcn_readfirstlane(tl * BN);
            if (kv0 < pg.n1) {
                issue_kv<C>(kbh, vbh, off, kv0, pg.n1, kslot(slot), vslot(slot), wave);
            } else {
                const size_t b2 = (size_t)bh * (Nkv - pg.n1) * D;
                issue_kv<C>((const char *)(pg.k2 + b2), (const char *)(pg.v2 + b2), off,
                            kv0 - pg.n1, Nkv - pg.n1, kslot(slot), vslot(slot), wave);
            }
        } else {
            issue_kv<C>(kbh, vbh, off, tl * BN, Nkv, kslot(slot), vslot(slot), wave);
        }
    };
    int kofs[C::NKK];
    const lds_char *vptr[C::NDB];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) kofs[kk] = li * C::ROWB + 16 * k_swz<D>(li, 2 * kk + g);
    {
        const int trow = 4 * g + ((lane & 15) >> 2);
        const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
            vptr[db] = (const lds_char *)(lds + C::VREG) + trow * C::ROWB +
                       16 * v_swz<D>(trow, 4 * db + tchunk) + 8 * (lane & 1);
    }

    // Prologue: tiles 0 .. NS-2 in flight; wait for tiles 0 and 1.
    TileSchedule::Cursor ld = sch.begin();
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
        if (j < ntl) {
            const int tl = MASK == kBlockSparse ? bs_tile(j) : ld.t;
            load_tile(tl, j);
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

    // The first tile's scores and their row maximum, which becomes the reference m.
    f32x16 sa, sb;
    float bnd = 0.f;
    int kv_cur = 0;  // first key of the tile the next step finishes (for its rare path)
    TileSchedule::Cursor nx = sch.begin();
    if (ntl > 0) {
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
            sa = Op::mma(*(const s16x8 *)(kslot(0) + kofs[kk]), qf[kk],
                         kk == 0 ? f32x16{} : sa);
        kv_cur = MASK == kBlockSparse ? tail_kv0 : nx.t * BN;
        if (nint == 0) mask_tile<MASK == kBlockSparse ? 0 : MASK>(sa, kv_cur, ip, Nkv, W, G, g);
        const float mt = half_swap_max(max16(sa)) * c;
        m = mt;
        nmu = mt == -INFINITY ? 0.f : -mt;
        bnd = mt == -INFINITY ? 0.f : sum_bound<T>();
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
            load_tile(tl, t + NS - 1);
            ld = sch.next(ld);
        }
    };
    // Steps come in pairs so that sa and sb swap roles without register copies, and the main
    // loop takes four at a time (the ring depth) so that each step's ring slots are known at
    // compile time and the LDS reads carry them as immediate offsets. Every step in the
    // loops has a tile t+1; the last step is peeled.
    auto step = [&](int t, f32x16 &cur, f32x16 &nxt) {
        load_ahead(t);
        const int kvn = MASK == kBlockSparse ? tail_kv0 : nx.t * BN;
        sp_step<T, C, MASK == kBlockSparse ? 0 : MASK, true>(
            kslot(t + 1), kslot(t), vring_ofs(t), kofs, vptr, qf, oacc, cur, nxt, m, nmu, bnd,
            l, c, t >= nint, kv_cur, t + 1 >= nint, kvn, ip, Nkv, W, G, g);
        kv_cur = kvn;
        nx = sch.next(nx);
        step_end(t);
    };
    auto last = [&](int t, f32x16 &cur, f32x16 &nxt) {
        sp_step<T, C, MASK == kBlockSparse ? 0 : MASK, false>(
            nullptr, kslot(t), vring_ofs(t), kofs, vptr, qf, oacc, cur, nxt, m, nmu, bnd, l, c,
            t >= nint, kv_cur, false, 0, ip, Nkv, W, G, g);
    };
    // Steady state (most steps): the step loads tile t + NS - 1, an interior tile (so its
    // index is found without walking the ranges), the next tile needs no element mask, and
    // the wait is for one tile in flight: no branches on any of these. The cursors are not
    // advanced here; the general loops below start from cursors set by position.
    auto steady = [&](int t, f32x16 &cur, f32x16 &nxt) {
        const int p = t + NS - 1;
        load_tile(MASK == kBlockSparse ? bs_tile(p) : sch.interior_tile(p), p);
        sp_step<T, C, MASK == kBlockSparse ? 0 : MASK, true>(
            kslot(t + 1), kslot(t), vring_ofs(t), kofs, vptr, qf, oacc, cur, nxt, m, nmu, bnd,
            l, c, false, 0, false, 0, ip, Nkv, W, G, g);
        wait_tiles<LPW, NS - 3>(NS - 3);
        ring_barrier();
    };
    if (ntl > 0) {
        int t = 0;
        for (; t + 3 + NS - 1 < nint; t += 4) {
            steady(t, sa, sb);
            steady(t + 1, sb, sa);
            steady(t + 2, sa, sb);
            steady(t + 3, sb, sa);
        }
        if (t > 0) {
            ld = sch.at(t + NS - 1);
            nx = sch.at(t + 1);
        }
        for (; t + 4 < ntl; t += 4) {
            step(t, sa, sb);
            step(t + 1, sb, sa);
            step(t + 2, sa, sb);
            step(t + 3, sb, sa);
        }
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
    // O leaves as whole rows through the idle K/V ring (32 rows per wave), when it fits.
    if constexpr (NW * 32 * (C::ROWB + 16) <= C::LDS_BYTES) {
        __syncthreads();  // every wave has finished reading K and V from the ring
        store_rows_via_lds<T, D>(lds + wave * 32 * (C::ROWB + 16), oacc, inv, lane,
                                 O + qbase, q0 + wave * 32, Nq, rs);
    } else if (row < Nq) {
        uint16_t *orow = O + qbase + (size_t)row * rs;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const s16x4 v4 = Op::pack4(oacc[db][4 * blk + 0] * inv, oacc[db][4 * blk + 1] * inv,
                                           oacc[db][4 * blk + 2] * inv, oacc[db][4 * blk + 3] * inv);
                *(s16x4 *)(orow + db * 32 + 8 * blk + 4 * g) = v4;
            }
        }
    }
    if (row < Nq && g == 0)
        LSE[lbase + (size_t)row * lstride] =
            lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
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

// 4 waves (128 query rows) per workgroup, two workgroups per CU, a 4-slot K/V ring: the
// fastest shape of a sweep over 2, 4 and 8 waves and 3 to 8 ring slots on MI355X. The sweep
// (tile_sweep.py) rebuilds with FA_FWD_WAVES and FA_FWD_STAGES set; the block-sparse kernel
// keeps 4 waves, since its query tile must match the 128-position layout block.
#ifndef FA_FWD_WAVES
#define FA_FWD_WAVES 4
#endif
#ifndef FA_FWD_STAGES
#define FA_FWD_STAGES 4
#endif
constexpr int kStages = FA_FWD_STAGES, kWaves = FA_FWD_WAVES;

template <typename T, int D, int MASK>
hipError_t launch16(const FwdArgs &a, hipStream_t s)
{
    constexpr int NS = MASK == kBlockSparse ? 4 : kStages, NW = MASK == kBlockSparse ? 4 : kWaves;
    using C = CfgSP<D, NS, NW>;
    const int nqt = (a.Nq + C::BM - 1) / C::BM;
    const long nblk = (long)nqt * a.B * a.H;
    auto kern = fwd16_kernel<T, D, MASK, NS, NW, kKvDense>;
    // block sparse: wave counts and the key-block list (2 bytes a block) after the ring
    const int lds = MASK == kBlockSparse ? C::LDS_BYTES + 16 + 2 * kMaxKeyBlocks : C::LDS_BYTES;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NT), lds, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (uint16_t *)a.o, a.lse, a.Nq, a.Nkv, a.scale * kLog2e, a.window,
                       a.n_global, nqt, a.layout, a.H, KvLayout{});
    return hipGetLastError();
}

// Chunked prefill against a paged cache: one workgroup per (sequence, head, 128-row tile of
// the longest chunk); workgroups past their own sequence's chunk return at once.
template <typename T, int D, int MASK>
hipError_t launch16_paged(const PrefillArgs &a, hipStream_t s)
{
    using C = CfgSP<D, kStages, kWaves>;
    const int nqt = (a.Qmax + C::BM - 1) / C::BM;
    const long nblk = (long)nqt * a.S * a.H;
    auto kern = fwd16_kernel<T, D, MASK, kStages, kWaves, kKvPaged>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    const KvLayout pg{a.page_table, a.seq_lens, a.q_lens, a.max_pages, a.num_pages, a.Qmax, a.H,
                      nullptr, nullptr, 0};
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NT), C::LDS_BYTES, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k_pages,
                       (const uint16_t *)a.v_pages, (uint16_t *)a.o, a.lse, 0, 0,
                       a.scale * kLog2e, a.window, a.n_global, nqt, nullptr, a.H, pg);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch16_paged_mask(const PrefillArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch16_paged<T, D, 0>(a, s);
    case 1: return launch16_paged<T, D, 1>(a, s);
    case 2: return launch16_paged<T, D, 2>(a, s);
    case 3: return launch16_paged<T, D, 3>(a, s);
    default: return launch16_paged<T, D, 4>(a, s);
    }
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

// Causal attention whose keys sit in two tensors (see KvLayout): [0, n1) in a.k/a.v,
// [n1, Nkv) in k2/v2.
template <typename T, int D>
hipError_t launch16_two_part(const FwdArgs &a, const void *k2, const void *v2, int n1,
                             hipStream_t s)
{
    using C = CfgSP<D, kStages, kWaves>;
    const int nqt = (a.Nq + C::BM - 1) / C::BM;
    const long nblk = (long)nqt * a.B * a.H;
    auto kern = fwd16_kernel<T, D, 1, kStages, kWaves, kKvTwoPart>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    KvLayout pg{};
    pg.k2 = (const uint16_t *)k2;
    pg.v2 = (const uint16_t *)v2;
    pg.n1 = n1;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NT), C::LDS_BYTES, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (uint16_t *)a.o, a.lse, a.Nq, a.Nkv, a.scale * kLog2e, 0, 0, nqt, nullptr,
                       a.H, pg);
    return hipGetLastError();
}

hipError_t launch_prefill_paged(const PrefillArgs &a, hipStream_t s)
{
    (void)hipGetLastError();
    if (a.dtype == 1)
        return a.d == 64 ? launch16_paged_mask<_Float16, 64>(a, s)
                         : launch16_paged_mask<_Float16, 128>(a, s);
    return a.d == 64 ? launch16_paged_mask<__bf16, 64>(a, s)
                     : launch16_paged_mask<__bf16, 128>(a, s);
}

hipError_t launch_forward_causal_two_part(const FwdArgs &a, const void *k2, const void *v2,
                                         int n1, hipStream_t s)
{
    (void)hipGetLastError();
    if (a.dtype == 1)
        return a.d == 64 ? launch16_two_part<_Float16, 64>(a, k2, v2, n1, s)
                         : launch16_two_part<_Float16, 128>(a, k2, v2, n1, s);
    return a.d == 64 ? launch16_two_part<__bf16, 64>(a, k2, v2, n1, s)
                     : launch16_two_part<__bf16, 128>(a, k2, v2, n1, s);
}

}  // namespace teaf
