// MALA backward, bf16 inputs, head dim 128, 128x64 tiles, on gfx950 MFMA.
//
// Source: "MassAlloc Attention: Let Attention Allocate Its Own Compute"
// (agihunt.info digest).  Backward paragraph: backward tests every legal tile
// against the FINAL log-normalizer written by forward (no stored mask, no
// replay of partial sums); the kept set is nested in forward's.  Motivation
// paragraph: backward post-score work is probability reconstruction plus dP,
// dS, dQ, dK and dV -- all of it is skipped for a skipped tile.
//
// Per tile (query block of 128 rows, key tile of 64 keys) the tile is kept
// iff some row i has a visible key j with s_ij - lse_i >= ln(tau) - ln(i+1),
// i.e. P_ij >= tau/Lq_i.  With thr_i = (lse_i*log2e + log2 tau - log2(i+1)) /
// (scale*log2e), computed once per row by bwd_prep, that is raw <q_i,k_j> >=
// thr_i.  Kept tiles:  P = exp(s - lse), dP = dO V^T, dS = P (dP - D),
// dV += P^T dO, dK += scale dS^T Q, dQ += scale dS K.
//
// Two kernels share the work:
//   dQ pass   -- one workgroup per query block (4 waves x 32 rows), scores
//                S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K, B = Q);
//                it tests every legal tile and writes the decision bits into
//                the backward's workspace;
//   dK/dV pass -- one workgroup per pair of 64-key tiles (8 waves), runs second and
//                visits only the query blocks those bits keep.
// No mask passes from forward to backward: the bits are made and consumed
// inside one mala_bwd call, from the final lse.
//
// Transposed operands (K^T for dQ, Q^T and dO^T for dK/dV) are read from the
// row-major LDS tiles with ds_read_b64_tr_b16: within each 16-lane group the
// 16 lanes read a 16x4 block M (one 8-byte row each) and lane i receives
// M[i/4 + 4e][i%4], e = 0..3 -- four consecutive rows at one column.
#include <float.h>

#include <type_traits>

#include "mala_kernels.hpp"

namespace mala {

namespace bwdk {
constexpr int BQ = 128, BK = 64, D = 128;
}  // namespace bwdk

// ------------------------------------------------------------------------- dQ
// One workgroup per query block (4 waves x 32 rows), key tiles from the
// diagonal back.  Backward thresholds depend only on the final lse, so the
// vote of a tile never waits for another tile's post-score work: while tile t
// is finished (its V in flight), the scores and the vote of tile t-1 are
// computed.  K tiles stream into a three-slot LDS ring two tiles ahead by
// direct global->LDS loads; V is requested right after a keep decision.
// Only the tiles at or past 2qb (the diagonal pair) need visibility masks;
// they are peeled off the loop as compile-time variants.
template <bool GATED, bool STATS>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    const float* __restrict__ thr, bf16_t* __restrict__ dq, int BH, int G, int L, int nqb, int words, float scale,
    float scale_log2, float log2_tau, int32_t* __restrict__ kept, int32_t* __restrict__ legal,
    uint32_t* __restrict__ bits, uint32_t* __restrict__ dbits, float* __restrict__ tstat) {
    using namespace bwdk;
    __shared__ __attribute__((aligned(1024))) uint8_t kring[3][BK * 256];
    __shared__ float tstat_sm[2][4];  // statistics only: each wave's largest test margin
    __shared__ __attribute__((aligned(1024))) uint8_t vtile[BK * 256];
    __shared__ int vote_sm[2][4];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    int qrank, bh;
    balanced_item(int(blockIdx.x), BH, max(1, nqb / 8), qrank, bh);
    const int qb = nqb - 1 - qrank;  // longest query blocks first
    const long hoff = long(bh) * L * D;       // this query head
    const long kvoff = long(bh / G) * L * D;  // its KV head (G query heads per KV head)
    const bf16_t* kh = k + kvoff;
    const bf16_t* vh = v + kvoff;
    const int row = qb * BQ + wave * 32 + j;
    const bool rvalid = row < L;

    // Q and dO rows as B operands; rows past L read row L-1 (their P is 0:
    // thr and lse are +inf there)
    u32x4 qf[8], of[8];
    const long rowc = min(row, L - 1);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        qf[s] = *reinterpret_cast<const u32x4*>(q + hoff + rowc * D + 16 * s + 8 * hl);
        of[s] = *reinterpret_cast<const u32x4*>(dout + hoff + rowc * D + 16 * s + 8 * hl);
    }
    const float th = rvalid ? thr[long(bh) * L + row] : INFINITY;
    const float l2 = rvalid ? lse2[long(bh) * L + row] : INFINITY;
    const float Di = rvalid ? Dv[long(bh) * L + row] : 0.f;

    f32x16 gacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) gacc[db][r] = 0.f;
    const int jmax = (min(qb * BQ + BQ, L) - 1) / BK;
    const int tdiag = 2 * qb;  // tiles t >= tdiag reach the diagonal

    // 64-row tile t -> 16 segments of 4 rows; wave w issues segments 4w..4w+3:
    // row 16w + 4it + l/16 of the tile, physical chunk l%16 (rows past L clamped).
    auto tile_dma = [&](const bf16_t* g, uint32_t la, int t) {
        la += 4096 * wave;
        const int rmax = L - 1 - t * BK;
        const bf16_t* gt = g + long(t) * BK * D;  // wave-uniform
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = 16 * wave + 4 * it + (lane >> 4);
            const uint32_t off = uint32_t(min(r, rmax) * D + (((lane & 15) ^ rowkey(r)) << 3)) * 2u;
            dma16s(gt, off, __builtin_amdgcn_readfirstlane(la + 1024 * it));
        }
    };
    int koff[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) koff[s] = swz(j, 2 * s + hl);
    int troff[4][2];
    tr_offsets(lane, troff);

    // S^T (keys x rows) of a tile: A = K rows from LDS, B = Q (registers).
    // The 16 products run from a register ring: the K operand of product i
    // (key block i & 1, step i >> 1) is read three products ahead, with a
    // scheduling fence after each product so that the reads stay ahead.
    auto scores = [&](uint32_t kb0, f32x16* sacc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        auto rd = [&](int i) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(lds_ptr(kb0 + 8192 * (i & 1)) + koff[i >> 1]);
        };
        u32x4 ring[4];
#pragma unroll
        for (int i = 0; i < 3; ++i) ring[i] = rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 3 < 16) ring[(i + 3) & 3] = rd(i + 3);
            __builtin_amdgcn_sched_barrier(0);
            sacc[i & 1] = mfma32(ring[i & 3], qf[i >> 1], sacc[i & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Scores of a tile at or past tdiag: keys past the row or past L become
    // -inf, so they neither vote nor carry probability.  Register r of key
    // block kb holds key t*64 + 32kb + 8(r/4) + 4hl + r%4.  Every key of a
    // tile below tdiag is visible to every row of the block.
    auto mask_diag = [&](int t, f32x16* sacc) {
        const int lim = min(row, L - 1) - t * BK - 4 * hl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
    };
    auto vote_of = [&](const f32x16* sacc) {
        bool vote = false;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) vote |= sacc[kb][r] >= th;
        return wave_any(vote);
    };

    // statistics: log2 of a tile's test statistic, the largest margin
    // c*(max_j s_ij - thr_i) = c*max_j s_ij - (lse2_i + log2 tau - log2 Lq_i) of
    // a voting row (rows without a visible key, and rows past L, abstain)
    auto margin_of = [&](const f32x16* sacc) -> float {
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        float dl = (mx == -INFINITY) ? -INFINITY : (mx - th) * scale_log2;
        if (row == 0 && mx != -INFINITY) dl = -log2_tau;  // row 0: P_00 = 1, T = 1/tau exactly
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) dl = fmaxf(dl, shfl_xor_f(dl, m));
        return dl;
    };
    const int ntk = (L + BK - 1) / BK;

    int nkept = 0;
    uint32_t word = 0;
    if (STATS && bits && tid == 0)
        for (int w = (jmax >> 5) + 1; w < words; ++w) bits[(long(bh) * nqb + qb) * words + w] = 0u;

    // K ring: tile t lives in kring[t % 3]
    const uint32_t vta = lds_addr_of(vtile);

    // prologue: K(jmax) (and K(jmax-1)) requested; scores + vote of tile jmax
    tile_dma(kh, lds_addr_of(kring[jmax % 3]), jmax);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    lds_barrier();
    if (jmax >= 1) tile_dma(kh, lds_addr_of(kring[(jmax + 2) % 3]), jmax - 1);
    f32x16 sc[2];  // scores of the tile being voted on
    scores(lds_addr_of(kring[jmax % 3]), sc);
    mask_diag(jmax, sc);
    if (GATED) {
        const bool wv = vote_of(sc);
        if (lane == 0) vote_sm[jmax & 1][wave] = wv ? 1 : 0;
        if (STATS && tstat) {
            const float dl = margin_of(sc);
            if (lane == 0) tstat_sm[jmax & 1][wave] = dl;
        }
    }

    // One step per tile; R = t % 3 is a compile-time constant, so the ring slot
    // addresses are constants (they fold into the instructions' offset fields).
    auto step = [&](auto res_tag, int t) {
        constexpr int R = decltype(res_tag)::value;
        const uint32_t ks0 = lds_addr_of(kring[R]);            // tile t
        const uint32_t ks1 = lds_addr_of(kring[(R + 2) % 3]);  // tile t-1
        const uint32_t ks2 = lds_addr_of(kring[(R + 1) % 3]);  // free: tile t-2 goes there
        // Everything issued in the previous step has landed: K(t-1) (and the
        // V tile that step consumed).
        __builtin_amdgcn_s_waitcnt(0x0f70);
        lds_barrier();  // vote flags of tile t and K(t-1) visible; previous V and K(t+1) reads done
        if (t >= 2) tile_dma(kh, ks2, t - 2);  // (independent of the vote: issued before its flags are read)
        int vflags = 1;
        if (GATED) vflags = vote_sm[t & 1][0] | vote_sm[t & 1][1] | vote_sm[t & 1][2] | vote_sm[t & 1][3];
        const bool keep = vflags != 0;
        if (keep) tile_dma(vh, vta, t);
        if (STATS && tstat && tid == 0)  // tau = 0 runs no test: NaN
            tstat[(long(bh) * nqb + qb) * ntk + t] =
                GATED ? fmaxf(fmaxf(tstat_sm[t & 1][0], tstat_sm[t & 1][1]), fmaxf(tstat_sm[t & 1][2], tstat_sm[t & 1][3]))
                      : NAN;
        // P = exp(s - lse) (zero on invisible entries) as bf16 B operands; step
        // (kb, hf) holds score registers 8hf .. 8hf+7 of key block kb
        u32x4 pk[2][2];
        if (keep) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r0 = 8 * hf + 2 * e;
                        pk[kb][hf][e] = pack_bf16x2(fast_exp2(fmaf(sc[kb][r0], scale_log2, -l2)),
                                                    fast_exp2(fmaf(sc[kb][r0 + 1], scale_log2, -l2)));
                    }
        }
        __builtin_amdgcn_sched_barrier(0);
        // scores and vote of the next tile while V(t) is in flight
        if (t >= 1) {
            scores(ks1, sc);
            if (t - 1 >= tdiag) mask_diag(t - 1, sc);
            if (GATED) {
                const bool wv = vote_of(sc);
                if (lane == 0) vote_sm[(t - 1) & 1][wave] = wv ? 1 : 0;
                if (STATS && tstat) {
                    const float dl = margin_of(sc);
                    if (lane == 0) tstat_sm[(t - 1) & 1][wave] = dl;
                }
            }
        }
        if (keep) {
            // K(t-2) and V(t) were issued at the start of the step; wait for both
            __builtin_amdgcn_s_waitcnt(0x0f70);
            lds_barrier();  // V(t) visible
            __builtin_amdgcn_sched_barrier(0);
            // per 32-key half kb: dP^T (keys x rows) = V dO^T; dS^T = P^T (dP^T - D)
            // (P from its bf16 operand copy, in place); dQ^T (d x rows) += K^T dS^T
            // with K^T read transposed from tile t's slot
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
                {  // V operands from a ring, three products ahead (as for the scores)
                    auto rd = [&](int s) -> u32x4 {
                        return *reinterpret_cast<const u32x4*>(lds_ptr(vta + 8192 * kb) + koff[s]);
                    };
                    u32x4 ring[4];
#pragma unroll
                    for (int s = 0; s < 3; ++s) ring[s] = rd(s);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        if (s + 3 < 8) ring[(s + 3) & 3] = rd(s + 3);
                        __builtin_amdgcn_sched_barrier(0);
                        pacc = mfma32(ring[s & 3], of[s], pacc);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r0 = 8 * hf + 2 * e;
                        const uint32_t w = pk[kb][hf][e];
                        pk[kb][hf][e] = pack_bf16x2(__uint_as_float(w << 16) * (pacc[r0] - Di),
                                                    __uint_as_float(w & 0xffff0000u) * (pacc[r0 + 1] - Di));
                    }
                __builtin_amdgcn_sched_barrier(0);
                {  // transposed K operands from a ring: product i = (db = i / 2, hf = i % 2)
                    auto rd = [&](int i) -> u32x4 {
                        return tr_operand_at(ks0 + 256 * (32 * kb + 16 * (i & 1)), troff[i >> 1]);
                    };
                    u32x4 ring[4];
#pragma unroll
                    for (int i = 0; i < 3; ++i) ring[i] = rd(i);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if (i + 3 < 8) ring[(i + 3) & 3] = rd(i + 3);
                        __builtin_amdgcn_sched_barrier(0);
                        gacc[i >> 1] = mfma32(ring[i & 3], pk[kb][i & 1], gacc[i >> 1]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        // decisions: handed to the dK/dV pass (dbits), and to the caller's stats
        if ((GATED || STATS) && tid == 0) {
            nkept += keep;
            if (keep) word |= 1u << (t & 31);
            if ((t & 31) == 0) {
                const long wi = (long(bh) * nqb + qb) * words + (t >> 5);
                if (GATED) dbits[wi] = word;
                if (STATS && bits) bits[wi] = word;
                word = 0;
            }
        }
    };

    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    using R2 = std::integral_constant<int, 2>;
    int t = jmax;
    if (t % 3 == 1) step(R1{}, t--);  // peel down to a tile with t % 3 == 2
    if (t % 3 == 0) step(R0{}, t--);
    for (; t >= 2; t -= 3) {
        step(R2{}, t);
        step(R1{}, t - 1);
        step(R0{}, t - 2);
    }

    if (rvalid) {
        bf16_t* grow = dq + hoff + long(row) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(gacc[db][4 * g + 0] * scale, gacc[db][4 * g + 1] * scale);
                w[1] = pack_bf16x2(gacc[db][4 * g + 2] * scale, gacc[db][4 * g + 3] * scale);
                *reinterpret_cast<u32x2*>(grow + 32 * db + 8 * g + 4 * hl) = w;
            }
    }
    if (STATS && tid == 0) {
        if (kept) kept[long(bh) * nqb + qb] = nkept;
        if (legal) legal[long(bh) * nqb + qb] = jmax + 1;
    }
}

// ---------------------------------------------------------------------- dK/dV
// Two layouts of the same pass.  Per workgroup: one 64-key tile
// (bwd_dkdv_tile_bf16_d128), or a pair of them (bwd_dkdv_pair_bf16_d128), which
// halves the Q/dO loads per FLOP but needs twice the work per workgroup; the
// launcher takes the pair layout when its grid still has at least two
// workgroups per CU.
//
// Tile layout.  One workgroup of 8 waves per 64-key tile: wave w owns keys 32(w&1) .. +31
// of the tile and rows 32(w>>1) .. +31 of every query block, so two waves
// share each SIMD.  K of the wave's keys is held in registers (B operand of
// S = Q K^T); the V tile sits in LDS (B operand of dP = dO V^T).
//
// Decisions.  The dQ pass runs first and tests every tile against the final
// lse; its decision bits reach this pass through the backward's workspace.
// This pass visits only the kept query blocks of its key tile: a skipped
// block costs no Q/dO load, no S and no post-score work, and both passes use
// the same decisions by construction.
//
// The Q and dO tiles of successive kept query blocks are double-buffered in
// LDS: while one block is computed, the next streams into the other buffer
// with direct global->LDS loads.  Each wave accumulates dK^T and dV^T over
// its own 32 rows of every block; the four row quarters are summed through
// LDS at the end.  Rows past L are read clamped to row L-1; their lse is
// +inf there, so P = 0.
template <bool GATED>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_tile_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int BHkv, int G, int L, int nqb, int words, float scale,
    float scale_log2, const uint32_t* __restrict__ dbits, uint32_t* __restrict__ aux_bits) {
    using namespace bwdk;
    // buf[0..3]: Q and dO tiles of two query blocks (buf[0], buf[1] and
    // buf[2], buf[3]); reused at the end for the cross-wave reduction.
    __shared__ __attribute__((aligned(1024))) uint8_t buf[4][BQ * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t vtile[BK * 256];
    __shared__ __attribute__((aligned(16))) float stA[2][BQ];  // lse2, D of the block's rows
    __shared__ __attribute__((aligned(16))) float stB[2][BQ];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    const int kb = wave & 1, rq = wave >> 1;
    int t, bkv;  // 64-key tile (longest, t = 0, first) and K/V head; its query heads are bkv*G .. +G-1
    balanced_item(int(blockIdx.x), BHkv, max(1, (2 * nqb) / 8), t, bkv);
    const long kvoff = long(bkv) * L * D;
    const int key = t * BK + 32 * kb + j;
    const bool kvalid = key < L;
    const int qb0 = (t * BK) / BQ;  // first query block that sees the tile (its diagonal block)
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    // K of this wave's 32 keys as B operands (lane = key, 8 contiguous d)
    u32x4 kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        kf[s] = kvalid ? *reinterpret_cast<const u32x4*>(k + kvoff + long(key) * D + 16 * s + 8 * hl) : z4;
    f32x16 dvacc[4], dkacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[db][r] = 0.f; dkacc[db][r] = 0.f; }

    // Direct loads of one 128x128 tile: 32 segments of 4 rows (1 KiB); wave w
    // issues segments 4w..4w+3 (rows 16w .. 16w+15); lane l of a segment fills
    // physical chunk l%16 of row l/16, i.e. it reads the logical chunk that the
    // swizzle puts there.  Rows past L read row L-1 instead (masked later).
    auto tile_async = [&](const bf16_t* g, uint8_t* dst, int bh, int r0) {
        const uint32_t la = lds_addr_of(dst) + 4096 * wave;
        const bf16_t* gb = g + long(bh) * L * D + long(r0) * D;  // wave-uniform
        const int lim = L - 1 - r0;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int rt = 16 * wave + 4 * it + (lane >> 4);
            const uint32_t off = uint32_t(min(rt, lim) * D + (((lane & 15) ^ rowkey(rt)) << 3)) * 2u;
            dma16s(gb, off, __builtin_amdgcn_readfirstlane(la + 1024 * it));
        }
    };
    // Operand read offsets within a Q or dO tile, this wave's row quarter
    // folded in: normal (row-major) reads of row 32rq + j, chunk 2s + hl, and
    // the transposed reads of tr_operand_at (rowbase 32rq).
    int qoff[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qoff[s] = swz(j, 2 * s + hl) + 8192 * rq;
    int troff[4][2];
    tr_offsets(lane, troff);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        troff[db][0] += 8192 * rq;
        troff[db][1] += 8192 * rq;
    }
    // Per-row state of a block, held by threads 0..127: loaded raw (row index
    // clamped) into registers before the tile prefetch is issued, written to
    // LDS (with the padding-row defaults) only at the end of the block, so
    // waiting for these loads never waits for the prefetch.
    float stv[2];
    int st_row = 0;
    auto stats_load = [&](int bh, int r0) {
        if (tid < BQ) {
            st_row = r0 + tid;
            const long ri = long(bh) * L + min(st_row, L - 1);
            stv[0] = lse2[ri];
            stv[1] = Dv[ri];
        }
    };
    auto stats_store = [&](float (*st)[BQ]) {
        if (tid < BQ) {
            const bool ok = st_row < L;
            st[0][tid] = ok ? stv[0] : INFINITY;
            st[1][tid] = ok ? stv[1] : 0.f;
        }
    };
    // this wave's 32 keys of V, addressed with the Q-tile offsets
    const uint32_t va = lds_addr_of(vtile) + 8192 * kb - 8192 * rq;

    // Work items are (query head of the group, kept query block), head by
    // head.  Kept blocks of one head come 64 at a time: bit i of kmask is
    // block wbase + i (every lane fetches one block's decision word, a ballot
    // packs the bits); the next window's words are fetched one window ahead.
    const uint32_t tbit = 1u << (t & 31);
    int ih = 0;  // query head within the group of the current window
    auto fetch = [&](int base) -> uint32_t {
        const int qb = base + lane;
        return (GATED && qb < nqb) ? dbits[(long(bkv * G + ih) * nqb + qb) * words + (t >> 5)] : 0u;
    };
    int wbase = qb0;
    uint64_t kmask = 0;
    uint32_t wnext = 0;
    auto open_head = [&]() {
        wbase = qb0;
        if (GATED) {
            kmask = __ballot((fetch(qb0) & tbit) != 0u);
            wnext = fetch(qb0 + 64);
        }
    };
    // first kept block >= qb (qb >= wbase) of head ih, or nqb
    auto kept_from = [&](int qb) -> int {
        if (!GATED) return qb;
        for (;;) {
            const int sh = qb - wbase;
            const uint64_t m = sh >= 64 ? 0ull : (kmask >> sh) << sh;
            if (m) return wbase + __builtin_ctzll(m);
            if (wbase + 64 >= nqb) return nqb;
            wbase += 64;
            qb = max(qb, wbase);
            kmask = __ballot((wnext & tbit) != 0u);
            wnext = fetch(wbase + 64);
        }
    };
    // the work item after (ih, qb): the next kept block of this head, else
    // the first kept block of the next head with one (ih == G: done)
    auto next_item = [&](int qb) -> int {
        int qn = kept_from(qb + 1);
        while (qn >= nqb && ih + 1 < G) {
            ++ih;
            open_head();
            qn = kept_from(qb0);
        }
        if (qn >= nqb) ih = G;
        return qn;
    };

    // One kept query block, computed from (qs, os, st).  Only the diagonal
    // block (qb == qb0) needs a visibility mask: it is the only block with
    // keys past some row, and the only block of the last tiles, whose keys may
    // run past L.  Elsewhere every key is visible to every row.
    auto block = [&](auto diag_tag, int bh, int qb, const uint8_t* qs, const uint8_t* os, const float (*st)[BQ]) {
        constexpr bool diag = decltype(diag_tag)::value;
        const int r0 = qb * BQ;
        const uint32_t qa = lds_addr_of(qs), oa = lds_addr_of(os);
        // S (32 rows x 32 keys) = Q K^T; register r holds row 32rq + 8(r/4) + 4hl + r%4, key j
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) sacc = mfma32(*reinterpret_cast<const u32x4*>(lds_ptr(qa) + qoff[s]), kf[s], sacc);
        if (diag) {  // keys past the row -> -inf: no probability
            const int lim = key - r0 - 32 * rq - 4 * hl;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) < lim) sacc[r] = -INFINITY;
        }
        __builtin_amdgcn_sched_barrier(0);
        // dP (32 rows x 32 keys) = dO V^T
        f32x16 pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            pacc = mfma32(*reinterpret_cast<const u32x4*>(lds_ptr(oa) + qoff[s]),
                          *reinterpret_cast<const u32x4*>(lds_ptr(va) + qoff[s]), pacc);
        __builtin_amdgcn_sched_barrier(0);
        // P = exp(s - lse) (zero where masked; lse2 = +inf on rows past L),
        // kept only as bf16 B operands: step hf holds registers 8hf .. 8hf+7.
        u32x4 pf[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 lz = *reinterpret_cast<const f32x4*>(&st[0][32 * rq + 8 * g + 4 * hl]);
            float p[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) p[x] = fast_exp2(fmaf(sacc[4 * g + x], scale_log2, -lz[x]));
            pf[g >> 1][2 * (g & 1)] = pack_bf16x2(p[0], p[1]);
            pf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(p[2], p[3]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // dV^T (d x keys) += dO^T P : A = dO^T (transposed read), B = P (lane = key)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                dvacc[db] = mfma32(tr_operand_at(oa + 256 * (16 * hf), troff[db]), pf[hf], dvacc[db]);
        __builtin_amdgcn_sched_barrier(0);
        // dS = P (dP - D), P taken from its bf16 operand copy
        u32x4 dsf[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 dd = *reinterpret_cast<const f32x4*>(&st[1][32 * rq + 8 * g + 4 * hl]);
            const uint32_t w0 = pf[g >> 1][2 * (g & 1)], w1 = pf[g >> 1][2 * (g & 1) + 1];
            const float p0 = __uint_as_float(w0 << 16), p1 = __uint_as_float(w0 & 0xffff0000u);
            const float p2 = __uint_as_float(w1 << 16), p3 = __uint_as_float(w1 & 0xffff0000u);
            dsf[g >> 1][2 * (g & 1)] = pack_bf16x2(p0 * (pacc[4 * g + 0] - dd[0]), p1 * (pacc[4 * g + 1] - dd[1]));
            dsf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(p2 * (pacc[4 * g + 2] - dd[2]), p3 * (pacc[4 * g + 3] - dd[3]));
        }
        __builtin_amdgcn_sched_barrier(0);
        // dK^T (d x keys) += Q^T dS
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                dkacc[db] = mfma32(tr_operand_at(qa + 256 * (16 * hf), troff[db]), dsf[hf], dkacc[db]);
        if (aux_bits && tid == 0)  // the blocks this pass visited (parity statistics)
            atomicOr(&aux_bits[(long(bh) * nqb + qb) * words + (t >> 5)], tbit);
    };

    // prologue: V tile; the first work item into buffers 0, 1
#pragma unroll
    for (int it = 0; it < 2; ++it) {  // V tile: segments 2w, 2w+1 (rows 8w .. 8w+7)
        const int rt = 8 * wave + 4 * it + (lane >> 4);
        const uint32_t off = uint32_t(min(rt, L - 1 - t * BK) * D + (((lane & 15) ^ rowkey(rt)) << 3)) * 2u;
        dma16s(v + kvoff + long(t) * BK * D, off,
               __builtin_amdgcn_readfirstlane(lds_addr_of(vtile) + 2048 * wave + 1024 * it));
    }
    open_head();
    int qb = kept_from(qb0);
    if (qb >= nqb) qb = next_item(nqb - 1);  // head 0 keeps nothing here: move on
    if (ih < G) {
        tile_async(q, buf[0], bkv * G + ih, qb * BQ);
        tile_async(dout, buf[1], bkv * G + ih, qb * BQ);
        stats_load(bkv * G + ih, qb * BQ);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    stats_store(stA);
    lds_barrier();
    // Each work item is computed from one buffer pair while the next streams
    // into the other.  A head's diagonal block, if kept, is its first item.
    bool odd = false;
    auto advance = [&](auto diag_tag) {
        const int bh = bkv * G + ih;
        const int qcur = qb;
        const int qn = next_item(qcur);
        const bool more = ih < G;
        if (more) {
            stats_load(bkv * G + ih, qn * BQ);
            tile_async(q, odd ? buf[0] : buf[2], bkv * G + ih, qn * BQ);
            tile_async(dout, odd ? buf[1] : buf[3], bkv * G + ih, qn * BQ);
        }
        block(diag_tag, bh, qcur, odd ? buf[2] : buf[0], odd ? buf[3] : buf[1], odd ? stB : stA);
        if (more) stats_store(odd ? stA : stB);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's loads into the next buffer landed
        lds_barrier();                       // next buffer complete; every wave is done with this one
        qb = qn;
        odd = !odd;
    };
    while (ih < G) {
        const int hcur = ih;
        if (qb == qb0) advance(std::true_type{});
        while (ih == hcur) advance(std::false_type{});
    }

    // Sum the four row quarters.  Accumulators hold dK^T, dV^T: lane = key,
    // register 4g + x of block db = d 32db + 8g + 4hl + x.  Wave w stores its
    // 16 (db, g) groups as float4 at red[(16w + 4db + g) * 64 + lane]; output
    // group gi = (kb, 4db + g, lane) sums waves kb, kb + 2, kb + 4, kb + 6.
    f32x4* red = reinterpret_cast<f32x4*>(&buf[0][0]);
    auto reduce_store = [&](const f32x16* acc, bf16_t* out, float mul) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                red[(16 * wave + 4 * db + g) * 64 + lane] =
                    f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gi = tid + 512 * i;
            const int l = gi & 63, dbg = (gi >> 6) & 15, kh = gi >> 10;
            f32x4 sum = red[(16 * kh + dbg) * 64 + l];
#pragma unroll
            for (int rr = 1; rr < 4; ++rr) {
                const f32x4 x = red[(16 * (kh + 2 * rr) + dbg) * 64 + l];
                sum[0] += x[0];
                sum[1] += x[1];
                sum[2] += x[2];
                sum[3] += x[3];
            }
            const int kk = t * BK + 32 * kh + (l & 31);
            if (kk < L) {
                u32x2 w;
                w[0] = pack_bf16x2(sum[0] * mul, sum[1] * mul);
                w[1] = pack_bf16x2(sum[2] * mul, sum[3] * mul);
                const int d0 = 32 * (dbg >> 2) + 8 * (dbg & 3) + 4 * (l >> 5);
                *reinterpret_cast<u32x2*>(out + kvoff + long(kk) * D + d0) = w;
            }
        }
        lds_barrier();
    };
    reduce_store(dkacc, dk, scale);
    reduce_store(dvacc, dv, 1.f);
}

// Pair layout.  One workgroup of 8 waves per pair of 64-key tiles (128 keys, tiles 2u and
// 2u+1): wave w owns keys 32kq .. +31 of the pair, kq = 2(w>>2) + (w&1) (so
// tile 2u + w/4), and rows 32((w>>1)&1) .. +31 of every 64-row half of a
// query block; waves w and w+4 share a SIMD.  The K and V tiles of the pair
// sit in LDS (B operands of S = Q K^T and dP = dO V^T); keys past L read key
// L-1 there, and the diagonal block's mask gives them no probability.
//
// Operand reads.  With the accumulators and the per-row state a wave is at
// the 256-register limit, and left to itself the compiler issues each LDS
// operand read just before its product, so every product waits out the LDS
// latency.  The products of a unit therefore run from explicit rings: the
// two operands of S and dP three products ahead, the transposed operands of
// dV and dK three ahead, with a scheduling fence after each product so the
// order stays; the rows' lse is read two products before P needs it.  K
// sits in LDS (not in registers) to make room for the rings.
//
// Decisions.  The dQ pass runs first and tests every tile against the final
// lse; its decision bits reach this pass through the backward's workspace.
// This pass visits the query blocks that keep at least one tile of its pair,
// and within a block the waves of a skipped tile do nothing: a block skipped
// by both tiles costs no Q/dO load, no S and no post-score work, and both
// passes use the same decisions by construction.
//
// A query block is processed in two 64-row halves, so one 16 KiB half of Q
// and of dO feeds 128 keys.  The halves of successive kept blocks are
// double-buffered in LDS: while one is computed, the next streams into the
// other buffer with direct global->LDS loads.  Each wave accumulates dK^T and
// dV^T over its 32 rows of every half; the two row groups are summed through
// LDS at the end.  Rows past L are read clamped to row L-1; their lse is +inf
// there, so P = 0, and a half with no row below L is not visited.
template <bool GATED>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int BHkv, int G, int L, int nqb, int words, float scale,
    float scale_log2, const uint32_t* __restrict__ dbits, uint32_t* __restrict__ aux_bits) {
    using namespace bwdk;
    constexpr int HB = 64, KP = 2 * BK;  // rows per half block, keys per workgroup
    // hbuf[0..3]: Q and dO halves of two work units (hbuf[0], hbuf[1] and
    // hbuf[2], hbuf[3]); reused at the end for the cross-wave reduction.
    __shared__ __attribute__((aligned(1024))) uint8_t hbuf[4][HB * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t vtile[KP * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t ktile[KP * 256];
    __shared__ __attribute__((aligned(16))) float stA[2][HB];  // lse2, D of the half's rows
    __shared__ __attribute__((aligned(16))) float stB[2][HB];

    const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar
    // waves w and w+4 share a SIMD and work on different tiles of the pair, so
    // a block that keeps one tile still has a wave on every SIMD
    const int tt = wave >> 2, kq = 2 * tt + (wave & 1), rh = (wave >> 1) & 1;
    int u, bkv;  // tile pair (longest, u = 0, first) and K/V head; its query heads are bkv*G .. +G-1
    balanced_item(int(blockIdx.x), BHkv, max(1, nqb / 8), u, bkv);
    const long kvoff = long(bkv) * L * D;
    const int key = u * KP + 32 * kq + j;
    const bool kvalid = key < L;
    const int qb0 = u;  // the pair's diagonal block: the first query block that sees it
    const bool t1 = 2 * u + 1 < (L + BK - 1) / BK;  // the pair's second tile exists

    f32x16 dvacc[4], dkacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[db][r] = 0.f; dkacc[db][r] = 0.f; }

    // Direct loads of one 64x128 half: 16 segments of 4 rows (1 KiB); wave w
    // issues segments 2w, 2w+1 (rows 8w .. 8w+7); lane l of a segment fills
    // physical chunk l%16 of row l/16, i.e. it reads the logical chunk that the
    // swizzle puts there.  Rows past L read row L-1 instead (r0 < L always).
    auto half_async = [&](const bf16_t* g, uint8_t* dst, int bh, int r0) {
        const uint32_t la = lds_addr_of(dst) + 2048 * wave;
        const bf16_t* gb = g + long(bh) * L * D + long(r0) * D;  // wave-uniform
        const int lim = L - 1 - r0;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int rt = 8 * wave + 4 * it + (lane >> 4);
            const uint32_t off = uint32_t(min(rt, lim) * D + (((lane & 15) ^ rowkey(rt)) << 3)) * 2u;
            dma16s(gb, off, __builtin_amdgcn_readfirstlane(la + 1024 * it));
        }
    };
    // Operand read offsets within a Q or dO half, this wave's row group folded
    // in: normal (row-major) reads of row 32rh + j, chunk 2s + hl, and the
    // transposed reads of tr_operand_at (rowbase 32rh).
    int qoff[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qoff[s] = swz(j, 2 * s + hl) + 8192 * rh;
    int troff[4][2];
    tr_offsets(lane, troff);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        troff[db][0] += 8192 * rh;
        troff[db][1] += 8192 * rh;
    }
    // Per-row state of a half, held by threads 0..63: loaded raw (row index
    // clamped) into registers before the next half's loads are issued, written
    // to LDS (with the padding-row defaults) only at the end of the unit, so
    // waiting for these loads never waits for the prefetch.
    float stv[2];
    int st_row = 0;
    auto stats_load = [&](int bh, int r0) {
        if (tid < HB) {
            st_row = r0 + tid;
            const long ri = long(bh) * L + min(st_row, L - 1);
            stv[0] = lse2[ri];
            stv[1] = Dv[ri];
        }
    };
    auto stats_store = [&](float (*st)[HB]) {
        if (tid < HB) {
            const bool ok = st_row < L;
            st[0][tid] = ok ? stv[0] : INFINITY;
            st[1][tid] = ok ? stv[1] : 0.f;
        }
    };
    // this wave's 32 keys of V, addressed with the Q-half offsets
    const uint32_t va = lds_addr_of(vtile) + 8192 * kq - 8192 * rh;
    const uint32_t ka = lds_addr_of(ktile) + 8192 * kq - 8192 * rh;

    // Work units are (query head of the group, kept query block, half),
    // head by head.  Kept blocks of one head come 64 at a time: bit i of km0
    // (km1) is block wbase + i keeping tile 2u (2u+1) -- every lane fetches
    // one block's decision word, ballots pack the bits; the next window's words
    // are fetched one window ahead.  Both tiles sit in one word.
    const int w0 = (2 * u) >> 5;
    const uint32_t bit0 = 1u << ((2 * u) & 31), bit1 = bit0 << 1;
    int ih = 0;  // query head within the group of the current window
    auto fetch = [&](int base) -> uint32_t {
        const int qb = base + lane;
        return (GATED && qb < nqb) ? dbits[(long(bkv * G + ih) * nqb + qb) * words + w0] : 0u;
    };
    int wbase = qb0;
    uint64_t km0 = 0, km1 = 0;
    uint32_t wnext = 0;
    auto load_window = [&](uint32_t w) {
        km0 = __ballot((w & bit0) != 0u);
        km1 = __ballot(t1 && (w & bit1) != 0u);
    };
    auto open_head = [&]() {
        wbase = qb0;
        if (GATED) {
            load_window(fetch(qb0));
            wnext = fetch(qb0 + 64);
        }
    };
    // first block >= qb (qb >= wbase) of head ih keeping a tile of the pair, or nqb
    auto kept_from = [&](int qb) -> int {
        if (!GATED) return qb;
        for (;;) {
            const int sh = qb - wbase;
            const uint64_t m = sh >= 64 ? 0ull : ((km0 | km1) >> sh) << sh;
            if (m) return wbase + __builtin_ctzll(m);
            if (wbase + 64 >= nqb) return nqb;
            wbase += 64;
            qb = max(qb, wbase);
            load_window(wnext);
            wnext = fetch(wbase + 64);
        }
    };
    // which tiles of the pair block qb keeps (bit 0: tile 2u, bit 1: 2u+1);
    // qb is in the current window
    auto flags_of = [&](int qb) -> int {
        if (!GATED) return t1 ? 3 : 1;
        const int sh = qb - wbase;
        return int((km0 >> sh) & 1ull) | (int((km1 >> sh) & 1ull) << 1);
    };
    // the block after (ih, qb) keeping a tile: the next one of this head, else
    // the first one of the next head with one (ih == G: done)
    auto next_item = [&](int qb) -> int {
        int qn = kept_from(qb + 1);
        while (qn >= nqb && ih + 1 < G) {
            ++ih;
            open_head();
            qn = kept_from(qb0);
        }
        if (qn >= nqb) ih = G;
        return qn;
    };

    // One unit: half h of block qb, computed from (qs, os, st).  Only the
    // diagonal block needs a visibility mask (keys past the row, including
    // keys past L); in its first half the second tile's keys lie past every
    // row, so those waves skip it.
    auto unit = [&](auto diag_tag, int bh, int qb, int h, int fl, const uint8_t* qs, const uint8_t* os,
                    const float (*st)[HB]) {
        constexpr bool diag = decltype(diag_tag)::value;
        if (aux_bits && tid == 0 && h == 0)  // the tiles this pass visits (parity statistics)
            atomicOr(&aux_bits[(long(bh) * nqb + qb) * words + w0], ((fl & 1) ? bit0 : 0u) | ((fl & 2) ? bit1 : 0u));
        if (!((fl >> tt) & 1)) return;        // this wave's tile is skipped for the block
        if (diag && h == 0 && kq >= 2) return;  // every key past every row of the half
        const int r0 = qb * BQ + HB * h;
        const uint32_t qa = lds_addr_of(qs), oa = lds_addr_of(os);
        // S (32 rows x 32 keys) = Q K^T and dP = dO V^T: 16 products whose two
        // operands are read from LDS three products ahead (a ring of four),
        // with a scheduling fence after each product so that the reads stay
        // ahead.  Register r of S holds row 32rh + 8(r/4) + 4hl + r%4, key j.
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
        auto rdA = [&](int i) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(lds_ptr(i < 8 ? qa : oa) + qoff[i & 7]);
        };
        auto rdB = [&](int i) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(lds_ptr(i < 8 ? ka : va) + qoff[i & 7]);
        };
        u32x4 ra[4], rb[4];
        f32x4 lz[4];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 3; ++i) { ra[i] = rdA(i); rb[i] = rdB(i); }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 3 < 16) { ra[(i + 3) & 3] = rdA(i + 3); rb[(i + 3) & 3] = rdB(i + 3); }
            if (i == 14) {  // the rows' lse for P, read while the last products run
#pragma unroll
                for (int g = 0; g < 4; ++g) lz[g] = *reinterpret_cast<const f32x4*>(&st[0][32 * rh + 8 * g + 4 * hl]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (i < 8) sacc = mfma32(ra[i & 3], rb[i & 3], sacc);
            else pacc = mfma32(ra[i & 3], rb[i & 3], pacc);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (diag) {  // keys past the row -> -inf: no probability
            const int lim = key - r0 - 32 * rh - 4 * hl;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) < lim) sacc[r] = -INFINITY;
        }
        __builtin_amdgcn_sched_barrier(0);
        // P = exp(s - lse) (zero where masked; lse2 = +inf on rows past L),
        // kept only as bf16 B operands: step hf holds registers 8hf .. 8hf+7.
        u32x4 pf[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float p[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) p[x] = fast_exp2(fmaf(sacc[4 * g + x], scale_log2, -lz[g][x]));
            pf[g >> 1][2 * (g & 1)] = pack_bf16x2(p[0], p[1]);
            pf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(p[2], p[3]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // transposed-operand products: product i = (db = i / 2, hf = i % 2),
        // A read three products ahead
        auto tr_pipe = [&](uint32_t base, const u32x4* bop, f32x16* acc) {
            u32x4 ta[4];
#pragma unroll
            for (int i = 0; i < 3; ++i) ta[i] = tr_operand_at(base + 256 * (16 * (i & 1)), troff[i >> 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i + 3 < 8) ta[(i + 3) & 3] = tr_operand_at(base + 256 * (16 * ((i + 3) & 1)), troff[(i + 3) >> 1]);
                __builtin_amdgcn_sched_barrier(0);
                acc[i >> 1] = mfma32(ta[i & 3], bop[i & 1], acc[i >> 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // dV^T (d x keys) += dO^T P : A = dO^T (transposed read), B = P (lane = key)
        __builtin_amdgcn_s_setprio(1);
        tr_pipe(oa, pf, dvacc);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        // dS = P (dP - D), P taken from its bf16 operand copy
        u32x4 dsf[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 dd = *reinterpret_cast<const f32x4*>(&st[1][32 * rh + 8 * g + 4 * hl]);
            const uint32_t w0p = pf[g >> 1][2 * (g & 1)], w1p = pf[g >> 1][2 * (g & 1) + 1];
            const float p0 = __uint_as_float(w0p << 16), p1 = __uint_as_float(w0p & 0xffff0000u);
            const float p2 = __uint_as_float(w1p << 16), p3 = __uint_as_float(w1p & 0xffff0000u);
            dsf[g >> 1][2 * (g & 1)] = pack_bf16x2(p0 * (pacc[4 * g + 0] - dd[0]), p1 * (pacc[4 * g + 1] - dd[1]));
            dsf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(p2 * (pacc[4 * g + 2] - dd[2]), p3 * (pacc[4 * g + 3] - dd[3]));
        }
        __builtin_amdgcn_sched_barrier(0);
        // dK^T (d x keys) += Q^T dS
        __builtin_amdgcn_s_setprio(1);
        tr_pipe(qa, dsf, dkacc);
        __builtin_amdgcn_s_setprio(0);
    };

    // prologue: K and V of the pair (segments 4w .. 4w+3, rows 16w .. 16w+15);
    // the first unit into buffers 0, 1
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int rt = 16 * wave + 4 * it + (lane >> 4);
        const uint32_t off = uint32_t(min(rt, L - 1 - u * KP) * D + (((lane & 15) ^ rowkey(rt)) << 3)) * 2u;
        dma16s(v + kvoff + long(u) * KP * D, off,
               __builtin_amdgcn_readfirstlane(lds_addr_of(vtile) + 4096 * wave + 1024 * it));
        dma16s(k + kvoff + long(u) * KP * D, off,
               __builtin_amdgcn_readfirstlane(lds_addr_of(ktile) + 4096 * wave + 1024 * it));
    }
    open_head();
    int qb = kept_from(qb0);
    if (qb >= nqb) qb = next_item(nqb - 1);  // head 0 keeps nothing here: move on
    int h = 0, fl = 0;
    if (ih < G) {
        fl = flags_of(qb);
        half_async(q, hbuf[0], bkv * G + ih, qb * BQ);
        half_async(dout, hbuf[1], bkv * G + ih, qb * BQ);
        stats_load(bkv * G + ih, qb * BQ);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    stats_store(stA);
    lds_barrier();
    // Each unit is computed from one buffer pair while the next streams into
    // the other.  A head's diagonal block, if kept, is its first block.
    bool odd = false;
    auto advance = [&](auto diag_tag) {
        const int bh = bkv * G + ih, qcur = qb, hcur = h, fcur = fl;
        if (h == 0 && qb * BQ + HB < L) {
            h = 1;  // second half of the same block
        } else {
            qb = next_item(qb);
            h = 0;
            if (ih < G) fl = flags_of(qb);
        }
        const bool more = ih < G;
        if (more) {
            const int r0n = qb * BQ + HB * h;
            stats_load(bkv * G + ih, r0n);
            half_async(q, odd ? hbuf[0] : hbuf[2], bkv * G + ih, r0n);
            half_async(dout, odd ? hbuf[1] : hbuf[3], bkv * G + ih, r0n);
        }
        unit(diag_tag, bh, qcur, hcur, fcur, odd ? hbuf[2] : hbuf[0], odd ? hbuf[3] : hbuf[1], odd ? stB : stA);
        if (more) stats_store(odd ? stA : stB);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's loads into the next buffers landed
        lds_barrier();                       // next buffers complete; every wave is done with these
        odd = !odd;
    };
    while (ih < G) {
        const int hcur = ih;
        while (ih == hcur && qb == qb0) advance(std::true_type{});  // at most its two halves
        while (ih == hcur) advance(std::false_type{});
    }

    // Sum the two row groups.  Accumulators hold dK^T, dV^T: lane = key,
    // register 4g + x of block db = d 32db + 8g + 4hl + x.  Waves of row group
    // 1 park theirs as float4 at red[(16kq + 4db + g) * 64 + lane]; the waves of
    // row group 0 with the same keys add them and write the result.
    f32x4* red = reinterpret_cast<f32x4*>(&hbuf[0][0]);
    auto reduce_store = [&](const f32x16* acc, bf16_t* out, float mul) {
        if (rh == 1) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    red[(16 * kq + 4 * db + g) * 64 + lane] =
                        f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        }
        lds_barrier();
        if (rh == 0 && kvalid) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 x = red[(16 * kq + 4 * db + g) * 64 + lane];
                    u32x2 w;
                    w[0] = pack_bf16x2((acc[db][4 * g] + x[0]) * mul, (acc[db][4 * g + 1] + x[1]) * mul);
                    w[1] = pack_bf16x2((acc[db][4 * g + 2] + x[2]) * mul, (acc[db][4 * g + 3] + x[3]) * mul);
                    // 32-bit element offset within the head (key < L): nothing
                    // per lane stays live from the start to here
                    *reinterpret_cast<u32x2*>(out + kvoff + uint32_t(key * D + 32 * db + 8 * g + 4 * hl)) = w;
                }
        }
        lds_barrier();
    };
    reduce_store(dkacc, dk, scale);
    reduce_store(dvacc, dv, 1.f);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
    const int BH = a.B * a.H;
    const int G = a.H / a.Hkv;  // query heads per K/V head (the API checked H % Hkv == 0)
    if (G < 1 || a.H % a.Hkv) return hipErrorInvalidValue;
    dim3 g2(unsigned(a.nqb) * unsigned(BH)), blk(256);
    const bool st = a.kept || a.legal || a.bits || a.tstat;
    hipError_t e = mark(a.ev[1], s);
    if (e != hipSuccess) return e;
#define MALA_DQ_LAUNCH(GT, ST)                                                                                \
    hipLaunchKernelGGL((bwd_dq_bf16_d128<GT, ST>), g2, blk, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,     \
                       (const bf16_t*)a.v, (const bf16_t*)a.dout, a.Dv, a.lse2, a.thr, (bf16_t*)a.dq, BH, G, a.L, \
                       a.nqb, a.words, a.scale, a.scale_log2, a.log2_tau, a.kept, a.legal, a.bits, a.dbits,    \
                       a.tstat)
    if (a.gated) {
        if (st) MALA_DQ_LAUNCH(true, true);
        else MALA_DQ_LAUNCH(true, false);
    } else {
        if (st) MALA_DQ_LAUNCH(false, true);
        else MALA_DQ_LAUNCH(false, false);
    }
#undef MALA_DQ_LAUNCH
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(a.ev[2], s);
    if (e != hipSuccess) return e;
    // pair layout when its grid keeps at least two workgroups per CU busy
    const bool pairs = long(a.nqb) * a.B * a.Hkv >= 2L * kNumCUs;
    const dim3 gk(unsigned(pairs ? a.nqb : a.ntiles) * unsigned(a.B * a.Hkv)), bk(512);
#define MALA_DKDV_LAUNCH(KERNEL, GT)                                                                           \
    hipLaunchKernelGGL((KERNEL<GT>), gk, bk, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, \
                       (const bf16_t*)a.dout, a.Dv, a.lse2, (bf16_t*)a.dk, (bf16_t*)a.dv, a.B * a.Hkv, G, a.L,    \
                       a.nqb, a.words, a.scale, a.scale_log2, a.dbits, a.aux_bits)
    if (pairs) {
        if (a.gated) MALA_DKDV_LAUNCH(bwd_dkdv_pair_bf16_d128, true);
        else MALA_DKDV_LAUNCH(bwd_dkdv_pair_bf16_d128, false);
    } else {
        if (a.gated) MALA_DKDV_LAUNCH(bwd_dkdv_tile_bf16_d128, true);
        else MALA_DKDV_LAUNCH(bwd_dkdv_tile_bf16_d128, false);
    }
#undef MALA_DKDV_LAUNCH
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(a.ev[3], s);
    return e;
}

}  // namespace mala
