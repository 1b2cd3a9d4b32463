// fa_bwd32.hip -- gradients of the float32 forward (dQ, dK, dV) for gfx950.
//
// The same recomputation as the 16-bit backward (the pages keep the N x N scores out of
// memory and rebuild them in the backward pass: ops-transformer article on gitcode.csdn.net,
// section 二.1; ascend-transformer-boost article, 场景一): with the forward's LSE,
// P = exp(scale Q K^T - LSE) is rebuilt tile by tile, and with D_i = dO_i . O_i
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   dK = scale dS^T Q,   dQ = scale dS K.
// The pages recommend fp32 or bf16 for training (ops-transformer article on
// gitcode.csdn.net, section 三.2 "精度与性能平衡"). These kernels take fp32 operands
// throughout (v_mfma_f32_32x32x2f32: true fp32 products, no rounding of P or dS) and, like
// the fp32 forward, are plain kernels: a parity path, not tuned beyond loading each tile
// one tile ahead (through registers into the second of two LDS stages).
//  * bwd32_dq_kernel runs first: a workgroup owns 128 query rows (4 waves x 32) with Q and
//    dO in registers, forms the row statistics (L_i = LSE_i log2 e, +inf for a row without
//    a visible key; D_i) and stores them per 32-row tile as [32 L, 32 -D] (the 16-bit
//    backward's workspace layout), then walks the visible 32-key tiles: S^T = K Q^T and
//    dP^T = V dO^T with lanes indexed by row, dQ^T += K^T dS^T.
//  * bwd32_dkdv_kernel: a workgroup owns 128 keys (4 waves x 32) with their K and V rows in
//    registers and walks the 32-row query tiles that can see them: S = Q K^T and
//    dP = dO V^T with lanes indexed by key, dV^T += dO^T P and dK^T += Q^T dS.
// Every sum runs in a fixed order with no atomics, so the results are reproducible.
#include "fa_bwd32.h"
#include "fa_device.h"

namespace teaf {
namespace {

// Rows and keys of a 32 x 32 fp32 MFMA result: lane (g, i) holds element e at position
// 8 (e / 4) + 4 g + e % 4 of the 32-long dimension (and i of the other).
__device__ __forceinline__ int mfma32_pos(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// Whether any query position in [ip0, ip1] sees any key in [k0, k1] under mask MASK (not
// the block-sparse layout, which is looked up per block).
template <int MASK>
__device__ __forceinline__ bool block_sees(int ip0, int ip1, int k0, int k1, int W, int G)
{
    if (MASK == 1) return ip1 >= k0;
    if (MASK == 2) return ip1 >= k0 && (k0 < G || ip0 - k1 < W);  // global or window key
    if (MASK == 3) return ip1 + W >= k0 && ip0 - W <= k1;
    if (MASK == 4) return k0 < G || ip1 >= k0;
    return true;
}

// Stores a 32 x D result held as D/32 transposed 32 x 32 fragments (lane (g, i): row i,
// columns db*32 + mfma32_pos(e, g)) times f into the row at out.
template <int D>
__device__ __forceinline__ void store_row(float *__restrict__ out, const f32x16 (&acc)[D / 32],
                                          float f, int g)
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const f32x4 v4 = {acc[db][4 * blk] * f, acc[db][4 * blk + 1] * f,
                              acc[db][4 * blk + 2] * f, acc[db][4 * blk + 3] * f};
            *(f32x4 *)(out + db * 32 + 8 * blk + 4 * g) = v4;
        }
}

template <int D, int MASK>
__global__ __launch_bounds__(256) void bwd32_dq_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ O, const float *__restrict__ LSE,
    float *__restrict__ st, float *__restrict__ dQ, int Nq, int Nkv, float c, float scale,
    int W, int G, int nqt, const uint8_t *__restrict__ layout, int H)
{
    constexpr int BM = 128, BN = 32, KP = D + 1, NKK = D / 2, NDB = D / 32;
    constexpr int RC = D / 4, CPT = BN * RC / 256;  // 16-byte pieces of a tile per thread
    constexpr int STAGE = 2 * BN * KP;              // one stage: the K rows, then the V rows
    extern __shared__ float stages[];               // two stages

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt, q0 = (L % nqt) * BM;
    const int delta = Nkv - Nq, nt32 = (Nq + 31) / 32;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;
    const int wrow0 = q0 + wave * 32, row = wrow0 + li, ip = row + delta;
    const bool live = row < Nq;

    // Q and dO as B operands (lane (g, i): row i, column 2 kk + g) and the row statistics.
    float qf[NKK], gf[NKK], dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const size_t at = qbase + (size_t)row * D + 2 * kk + g;
        qf[kk] = live ? Q[at] : 0.f;
        gf[kk] = live ? dO[at] : 0.f;
        dpart += live ? gf[kk] * O[at] : 0.f;
    }
    const float Drow = dpart + __shfl_xor(dpart, 32);
    const float lse = live ? LSE[(size_t)bh * Nq + row] : -INFINITY;
    const float Lrow = lse == -INFINITY ? INFINITY : lse * kLog2e;
    if (wrow0 < Nq) st[((size_t)bh * nt32 + wrow0 / 32) * 64 + 32 * g + li] = g ? -Drow : Lrow;

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;

    const TileRanges tr = visible_tiles<MASK, BM, BN>(q0, Nq, Nkv, W, G);
    const int na = tr.a1 - tr.a0, ntiles = na + (tr.b1 - tr.b0);
    const uint8_t *lrow = nullptr;
    if (MASK == kBlockSparse) {
        const int nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        lrow = layout + ((size_t)(bh % H) * nqt + q0 / kSparseBlock) * nkb;
    }
    auto tile_of = [&](int n) { return n < na ? tr.a0 + n : tr.b0 + (n - na); };
    // The first tile position at or after n that the workgroup visits (block sparse: the
    // key blocks its layout row marks visible).
    auto next_tile = [&](int n) {
        if (MASK == kBlockSparse)
            while (n < ntiles && lrow[tile_of(n) * BN / kSparseBlock] == 0) ++n;
        return n;
    };
    // A tile's K and V rows go to registers one tile ahead (their loads in flight during the
    // current tile's products), then into the other LDS stage; keys at or past Nkv are zero.
    f32x4 kpre[CPT], vpre[CPT];
    auto fetch = [&](int n) {
        const int kv0 = tile_of(n) * BN;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int id = tid + u * 256, r = id / RC, cc = id % RC;
            const size_t at = kvbase + (size_t)(kv0 + r) * D + 4 * cc;
            const bool in = kv0 + r < Nkv;
            kpre[u] = in ? *(const f32x4 *)(K + at) : f32x4{0.f, 0.f, 0.f, 0.f};
            vpre[u] = in ? *(const f32x4 *)(V + at) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto stash = [&](float *sk) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int id = tid + u * 256, r = id / RC, cc = id % RC;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk[r * KP + 4 * cc + e] = kpre[u][e];
                sk[BN * KP + r * KP + 4 * cc + e] = vpre[u][e];
            }
        }
    };
    int n = next_tile(0), stage = 0;
    if (n < ntiles) {
        fetch(n);
        stash(stages);
    }
    __syncthreads();
    while (n < ntiles) {
        const int kv0 = tile_of(n) * BN, nn = next_tile(n + 1);
        if (nn < ntiles) fetch(nn);
        const float *ks = stages + stage * STAGE, *vs = ks + BN * KP;
        if (wrow0 < Nq &&
            (MASK == 0 || MASK == kBlockSparse ||
             block_sees<MASK>(wrow0 + delta, wrow0 + 31 + delta, kv0, kv0 + BN - 1, W, G))) {
            f32x16 s, dp;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[li * KP + 2 * kk + g], qf[kk], s, 0,
                                                         0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[li * KP + 2 * kk + g], gf[kk], dp,
                                                          0, 0, 0);
            }
            // dS^T in place of S^T: lane (g, i) holds keys kv0 + mfma32_pos(e, g) of row i.
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kv0 + mfma32_pos(e, g);
                const bool vis = key < Nkv && key_visible<MASK>(ip, key, W, G);
                const float p = vis ? fast_exp2(s[e] * c - Lrow) : 0.f;
                s[e] = p * (dp[e] - Drow);
            }
            // dQ^T += K^T dS^T, one key per lane half and step.
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int kr = mfma32_pos(e, g);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dq[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[kr * KP + db * 32 + li],
                                                                  s[e], dq[db], 0, 0, 0);
            }
        }
        if (nn < ntiles) stash(stages + (stage ^ 1) * STAGE);
        __syncthreads();  // the next stage is written, this one's readers are done
        stage ^= 1;
        n = nn;
    }
    if (live) store_row<D>(dQ + qbase + (size_t)row * D, dq, scale, g);
}

template <int D, int MASK>
__global__ __launch_bounds__(256) void bwd32_dkdv_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ st, float *__restrict__ dK,
    float *__restrict__ dV, int Nq, int Nkv, float c, float scale, int W, int G, int nkt,
    const uint8_t *__restrict__ layout, int H)
{
    constexpr int BK = 128, KP = D + 1, NKK = D / 2, NDB = D / 32;
    static_assert(BK == kSparseBlock, "a workgroup's keys are one block of the sparse layout");
    constexpr int RC = D / 4, CPT = 32 * RC / 256;  // 16-byte pieces of a tile per thread
    constexpr int STAGE = 2 * 32 * KP + 64;  // Q rows, dO rows, the tile's L then -D values
    extern __shared__ float stages[];        // two stages

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nkt, k0 = (L % nkt) * BK;
    const int delta = Nkv - Nq, nt32 = (Nq + 31) / 32;
    const size_t qbase = (size_t)bh * Nq * D, kvbase = (size_t)bh * Nkv * D;
    const int wk0 = k0 + wave * 32, key = wk0 + li;
    const bool live = key < Nkv;

    // K and V as B operands (lane (g, i): key i, column 2 kk + g).
    float kf[NKK], vf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const size_t at = kvbase + (size_t)key * D + 2 * kk + g;
        kf[kk] = live ? K[at] : 0.f;
        vf[kk] = live ? V[at] : 0.f;
    }
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.f;

    const uint8_t *lcol = nullptr;  // the layout's column of this key block (stride nkb)
    int nkb = 0;
    if (MASK == kBlockSparse) {
        const int nqb = (Nq + kSparseBlock - 1) / kSparseBlock;
        nkb = (Nkv + kSparseBlock - 1) / kSparseBlock;
        lcol = layout + (size_t)(bh % H) * nqb * nkb + k0 / kSparseBlock;
    }
    const int kend = min(k0 + BK, Nkv) - 1;
    // Whether the workgroup visits 32-row tile t, and the first such tile at or after t.
    auto visits = [&](int t) {
        const int r0 = 32 * t;
        if (MASK == kBlockSparse) return lcol[(size_t)(r0 / kSparseBlock) * nkb] != 0;
        return MASK == 0 ||
               block_sees<MASK>(r0 + delta, min(r0 + 31, Nq - 1) + delta, k0, kend, W, G);
    };
    auto next_tile = [&](int t) {
        while (t < nt32 && !visits(t)) ++t;
        return t;
    };
    // A tile's Q and dO rows and its statistics go to registers one tile ahead (their loads in
    // flight during the current tile's products), then into the other LDS stage; rows at or
    // past Nq are zero.
    f32x4 qpre[CPT], gpre[CPT];
    float spre = 0.f;
    auto fetch = [&](int t) {
        const int r0 = 32 * t;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int id = tid + u * 256, r = id / RC, cc = id % RC;
            const size_t at = qbase + (size_t)(r0 + r) * D + 4 * cc;
            const bool in = r0 + r < Nq;
            qpre[u] = in ? *(const f32x4 *)(Q + at) : f32x4{0.f, 0.f, 0.f, 0.f};
            gpre[u] = in ? *(const f32x4 *)(dO + at) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (tid < 64) spre = st[((size_t)bh * nt32 + t) * 64 + tid];
    };
    auto stash = [&](float *sg) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int id = tid + u * 256, r = id / RC, cc = id % RC;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sg[r * KP + 4 * cc + e] = qpre[u][e];
                sg[32 * KP + r * KP + 4 * cc + e] = gpre[u][e];
            }
        }
        if (tid < 64) sg[2 * 32 * KP + tid] = spre;
    };
    int t = next_tile(0), stage = 0;
    if (t < nt32) {
        fetch(t);
        stash(stages);
    }
    __syncthreads();
    while (t < nt32) {
        const int r0 = 32 * t, tn = next_tile(t + 1);
        if (tn < nt32) fetch(tn);
        const float *qs = stages + stage * STAGE, *gs = qs + 32 * KP, *stat = gs + 32 * KP;
        if (wk0 < Nkv) {
            f32x16 s, dp;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[li * KP + 2 * kk + g], kf[kk], s, 0,
                                                         0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[li * KP + 2 * kk + g], vf[kk], dp,
                                                          0, 0, 0);
            }
            // P and dS: lane (g, i) holds rows r0 + mfma32_pos(e, g) of key i.
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = mfma32_pos(e, g), rw = r0 + r;
                const bool vis = live && rw < Nq && key_visible<MASK>(rw + delta, key, W, G);
                const float p = vis ? fast_exp2(s[e] * c - stat[r]) : 0.f;
                s[e] = p;
                dp[e] = p * (dp[e] + stat[32 + r]);
            }
            // dV^T += dO^T P and dK^T += Q^T dS, one row per lane half and step.
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = mfma32_pos(e, g);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[r * KP + db * 32 + li],
                                                                  s[e], dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[r * KP + db * 32 + li],
                                                                  dp[e], dk[db], 0, 0, 0);
                }
            }
        }
        if (tn < nt32) stash(stages + (stage ^ 1) * STAGE);
        __syncthreads();  // the next stage is written, this one's readers are done
        stage ^= 1;
        t = tn;
    }
    if (live) {
        store_row<D>(dK + kvbase + (size_t)key * D, dk, scale, g);
        store_row<D>(dV + kvbase + (size_t)key * D, dv, 1.f, g);
    }
}

template <int D, int MASK>
hipError_t launch_bwd32(const BwdArgs &a, hipStream_t s)
{
    const float c = a.scale * kLog2e;
    const int nqt = (a.Nq + 127) / 128, nkt = (a.Nkv + 127) / 128;
    // dQ first: it also writes the row statistics the dK/dV kernel reads. Its two LDS stages
    // of K and V rows take 66 KB at d 128.
    constexpr int lds_dq = 2 * 2 * 32 * (D + 1) * (int)sizeof(float);
    auto kq = bwd32_dq_kernel<D, MASK>;
    hipError_t e = hipFuncSetAttribute((const void *)kq,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_dq);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kq, dim3((unsigned)((long)nqt * a.B * a.H)),
                       dim3(256), lds_dq, s, (const float *)a.q, (const float *)a.k,
                       (const float *)a.v, (const float *)a.dout, (const float *)a.o, a.lse,
                       (float *)a.workspace, (float *)a.dq, a.Nq, a.Nkv, c, a.scale, a.window,
                       a.n_global, nqt, a.layout, a.H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int lds_dkdv = 2 * (2 * 32 * (D + 1) + 64) * (int)sizeof(float);
    auto kkv = bwd32_dkdv_kernel<D, MASK>;
    e = hipFuncSetAttribute((const void *)kkv, hipFuncAttributeMaxDynamicSharedMemorySize,
                            lds_dkdv);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kkv, dim3((unsigned)((long)nkt * a.B * a.H)),
                       dim3(256), lds_dkdv, s, (const float *)a.q, (const float *)a.k,
                       (const float *)a.v, (const float *)a.dout, (const float *)a.workspace,
                       (float *)a.dk, (float *)a.dv, a.Nq, a.Nkv, c, a.scale, a.window,
                       a.n_global, nkt, a.layout, a.H);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd32_mask(const BwdArgs &a, hipStream_t s)
{
    switch (a.mask) {
    case 0: return launch_bwd32<D, 0>(a, s);
    case 1: return launch_bwd32<D, 1>(a, s);
    case 2: return launch_bwd32<D, 2>(a, s);
    case 3: return launch_bwd32<D, 3>(a, s);
    case 4: return launch_bwd32<D, 4>(a, s);
    default: return launch_bwd32<D, kBlockSparse>(a, s);
    }
}

}  // namespace

hipError_t launch_backward32(const BwdArgs &a, hipStream_t s)
{
    (void)hipGetLastError();
    return a.d == 64 ? launch_bwd32_mask<64>(a, s) : launch_bwd32_mask<128>(a, s);
}

}  // namespace teaf
