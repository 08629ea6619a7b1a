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
// Two kernels share the work and take the SAME decisions without exchanging
// any mask:
//   dQ pass   -- one workgroup per query block (4 waves x 32 rows), scores
//                S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K, B = Q);
//   dK/dV pass -- one workgroup per 128 keys (4 waves x 32 keys, i.e. two
//                key tiles), scores S = Q K^T with the same instruction and
//                the same k-step order (A = Q, B = K).
// MFMA computes each output element as the same ordered sum over k whichever
// operand holds which matrix, so both passes see bit-identical raw scores and
// compare them with the same per-row threshold.
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
template <bool GATED, bool STATS>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    const float* __restrict__ thr, bf16_t* __restrict__ dq, int BH, int L, int nqb, int words, float scale,
    float scale_log2, int32_t* __restrict__ kept, int32_t* __restrict__ legal, uint32_t* __restrict__ bits) {
    using namespace bwdk;
    __shared__ __attribute__((aligned(1024))) uint8_t kring[3][BK * 256];  // K tile t in kring[t % 3]
    __shared__ __attribute__((aligned(1024))) uint8_t vtile[BK * 256];
    __shared__ int vote_sm[2][4];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    const int qb = nqb - 1 - int(blockIdx.x) / BH;
    const int bh = int(blockIdx.x) % BH;
    const long hoff = long(bh) * L * D;
    const bf16_t* kh = k + hoff;
    const bf16_t* vh = v + hoff;
    const int row = qb * BQ + wave * 32 + j;
    const bool rvalid = row < L;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    u32x4 qf[8], of[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        qf[s] = rvalid ? *reinterpret_cast<const u32x4*>(q + hoff + long(row) * D + 16 * s + 8 * hl) : z4;
        of[s] = rvalid ? *reinterpret_cast<const u32x4*>(dout + hoff + long(row) * D + 16 * s + 8 * hl) : z4;
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

    // 64-row tile t -> 16 segments of 4 rows; wave w issues segments 4w..4w+3:
    // row 16w + 4it + l/16 of the tile, physical chunk l%16 (rows past L clamped).
    const int drow = 16 * wave + (lane >> 4);
    const int dchk = (lane & 15) << 3;
    auto tile_dma = [&](const bf16_t* g, uint8_t* dst, int t) {
        const uint32_t la = lds_addr_of(dst) + 4096 * wave;
        const int rmax = L - 1 - t * BK;
        const bf16_t* gt = g + long(t) * BK * D;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = drow + 4 * it;
            dma16(gt + min(r, rmax) * D + (dchk ^ (rowkey(r) << 3)), __builtin_amdgcn_readfirstlane(la + 1024 * it));
        }
    };
    int koff[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) koff[s] = swz(j, 2 * s + hl);
    int troff[4][2];
    tr_offsets(lane, troff);

    // S^T (keys x rows) of a tile: A = K rows from LDS, B = Q (registers)
    auto scores = [&](const uint8_t* kt, f32x16* sacc) {
        const uint32_t kb0 = lds_addr_of(kt);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(lds_ptr(kb0 + 8192 * kb) + koff[s]);
                sacc[kb] = mfma32(a, qf[s], sacc[kb]);
            }
        }
    };
    // visibility (causal, in range) of register r of key block kb on tile t
    auto visible = [&](int t, int kb, int r) {
        const int key = t * BK + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
        return t < 2 * qb || (key <= row && key < L);
    };
    auto vote_of = [&](int t, const f32x16* sacc) {
        bool vote = false;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) vote |= visible(t, kb, r) && sacc[kb][r] >= th;
        return wave_any(vote);
    };

    int nkept = 0;
    uint32_t word = 0;
    if (STATS && bits && tid == 0)
        for (int w = (jmax >> 5) + 1; w < words; ++w) bits[(long(bh) * nqb + qb) * words + w] = 0u;

    // prologue: K(jmax) (and K(jmax-1)) requested; scores + vote of tile jmax
    tile_dma(kh, kring[jmax % 3], jmax);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    lds_barrier();
    if (jmax >= 1) tile_dma(kh, kring[(jmax - 1) % 3], jmax - 1);
    f32x16 sc[2];  // scores of the tile being voted on
    scores(kring[jmax % 3], sc);
    if (GATED) {
        const bool wv = vote_of(jmax, sc);
        if (lane == 0) vote_sm[jmax & 1][wave] = wv ? 1 : 0;
    }

    for (int t = jmax; t >= 0; --t) {
        // Everything issued in the previous iteration has landed: K(t-1) (and
        // the V tile that iteration consumed).
        __builtin_amdgcn_s_waitcnt(0x0f70);
        lds_barrier();  // vote flags of tile t and K(t-1) visible; previous V reads done
        int vflags = 1;
        if (GATED) vflags = vote_sm[t & 1][0] | vote_sm[t & 1][1] | vote_sm[t & 1][2] | vote_sm[t & 1][3];
        const bool keep = vflags != 0;
        if (keep) tile_dma(vh, vtile, t);
        if (t >= 2) tile_dma(kh, kring[(t - 2) % 3], t - 2);
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
                        const float p0 = visible(t, kb, r0) ? fast_exp2(fmaf(sc[kb][r0], scale_log2, -l2)) : 0.f;
                        const float p1 =
                            visible(t, kb, r0 + 1) ? fast_exp2(fmaf(sc[kb][r0 + 1], scale_log2, -l2)) : 0.f;
                        pk[kb][hf][e] = pack_bf16x2(p0, p1);
                    }
        }
        __builtin_amdgcn_sched_barrier(0);
        // scores and vote of the next tile while V(t) is in flight
        if (t >= 1) {
            scores(kring[(t - 1) % 3], sc);
            if (GATED) {
                const bool wv = vote_of(t - 1, sc);
                if (lane == 0) vote_sm[(t - 1) & 1][wave] = wv ? 1 : 0;
            }
        }
        if (keep) {
            // V(t) was issued just before K(t-2); wait for both (this kernel may
            // also have register-spill traffic in flight, so no partial counts)
            __builtin_amdgcn_s_waitcnt(0x0f70);
            lds_barrier();  // V(t) visible
            __builtin_amdgcn_sched_barrier(0);
            // dP^T (keys x rows) = V dO^T
            f32x16 pacc[2];
            const uint32_t vb0 = lds_addr_of(vtile);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) pacc[kb][r] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(lds_ptr(vb0 + 8192 * kb) + koff[s]);
                    pacc[kb] = mfma32(a, of[s], pacc[kb]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // dS^T = P^T (dP^T - D), P taken from its bf16 operand copy, in place
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r0 = 8 * hf + 2 * e;
                        const uint32_t w = pk[kb][hf][e];
                        pk[kb][hf][e] = pack_bf16x2(__uint_as_float(w << 16) * (pacc[kb][r0] - Di),
                                                    __uint_as_float(w & 0xffff0000u) * (pacc[kb][r0 + 1] - Di));
                    }
            __builtin_amdgcn_sched_barrier(0);
            // dQ^T (d x rows) += K^T dS^T ; K^T read transposed from tile t's slot
            const uint32_t kt0 = lds_addr_of(kring[t % 3]);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        gacc[db] = mfma32(tr_operand_at(kt0 + 256 * (32 * kb + 16 * hf), troff[db]), pk[kb][hf],
                                          gacc[db]);
        }
        if (STATS && tid == 0) {
            nkept += keep;
            if (keep) word |= 1u << (t & 31);
            if (bits && (t & 31) == 0) {
                bits[(long(bh) * nqb + qb) * words + (t >> 5)] = word;
                word = 0;
            }
        }
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
// One workgroup per 128 keys.  The Q and dO tiles of successive query blocks
// are double-buffered in LDS: while block qb is being computed from one
// buffer, block qb+1 streams into the other with direct global->LDS loads
// (no registers involved).  Rows past L are read clamped to row L-1 and are
// masked out of every vote and every product (P = 0 there).
template <bool GATED>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    const float* __restrict__ thr, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int BH, int L, int nqb,
    int ncol, int words, float scale, float scale_log2, uint32_t* __restrict__ aux_bits) {
    using namespace bwdk;
    __shared__ __attribute__((aligned(1024))) uint8_t qsA[BQ * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t osA[BQ * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t qsB[BQ * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t osB[BQ * 256];
    __shared__ __attribute__((aligned(16))) float stA[3][BQ];  // thr, lse2, D of the block's rows
    __shared__ __attribute__((aligned(16))) float stB[3][BQ];
    __shared__ int vote_sm[2][4];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    const int c = int(blockIdx.x) / BH;  // 128-key column; longest (c = 0) first
    const int bh = int(blockIdx.x) % BH;
    const long hoff = long(bh) * L * D;
    const int key = 128 * c + 32 * wave + j;
    const bool kvalid = key < L;
    const int tw = 2 * c + (wave >> 1);  // this wave's key tile
    const bool tile_exists = tw * BK < L;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    (void)ncol;

    // K and V of this wave's 32 keys as B operands (lane = key, 8 contiguous d)
    u32x4 kf[8], vf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        kf[s] = kvalid ? *reinterpret_cast<const u32x4*>(k + hoff + long(key) * D + 16 * s + 8 * hl) : z4;
        vf[s] = kvalid ? *reinterpret_cast<const u32x4*>(v + hoff + long(key) * D + 16 * s + 8 * hl) : z4;
    }
    f32x16 dvacc[4], dkacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[db][r] = 0.f; dkacc[db][r] = 0.f; }

    // Direct loads of one 128x128 tile: 32 segments of 4 rows (1 KiB); wave w
    // issues segments 8w..8w+7; lane l of a segment fills physical chunk l%16
    // of row l/16, i.e. it reads the logical chunk that the swizzle puts there.
    // Per-lane source offsets are fixed; rows past L are clamped on the last
    // block only.  Completion is awaited explicitly at the end of the block.
    int gofs[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int rt = 4 * it + (lane >> 4);
        gofs[it] = (32 * wave + rt) * D + (((lane & 15) ^ rowkey(rt)) << 3);
    }
    auto tile_async = [&](const bf16_t* g, uint8_t* dst, int r0) {
        const uint32_t la = lds_addr_of(dst) + 8192 * wave;
        if (r0 + BQ <= L) {
            const bf16_t* gt = g + hoff + long(r0) * D;
#pragma unroll
            for (int it = 0; it < 8; ++it) dma16(gt + gofs[it], __builtin_amdgcn_readfirstlane(la + 1024 * it));
        } else {
#pragma unroll
            for (int it = 0; it < 8; ++it) dma_segment(g + hoff, r0, L - r0, dst, 8 * wave + it, lane);
        }
    };
    int qoff[8];  // normal (row-major) operand reads: row j of a 32-row block, chunk 2s + hl
#pragma unroll
    for (int s = 0; s < 8; ++s) qoff[s] = swz(j, 2 * s + hl);
    int troff[4][2];
    tr_offsets(lane, troff);
    // Per-row state of a block: loaded raw (row index clamped) into registers
    // before the tile prefetch is issued, written to LDS (with the padding-row
    // defaults) only at the end of the iteration, so waiting for these loads
    // never waits for the prefetch.
    float stv[3];
    int st_row = 0;
    auto stats_load = [&](int r0) {
        st_row = r0 + (tid & (BQ - 1));
        const long ri = long(bh) * L + min(st_row, L - 1);
        stv[0] = thr[ri];
        stv[1] = lse2[ri];
        stv[2] = Dv[ri];
    };
    auto stats_store = [&](float (*st)[BQ]) {
        if (tid < BQ) {
            const bool ok = st_row < L;
            st[0][tid] = ok ? stv[0] : INFINITY;
            st[1][tid] = ok ? stv[1] : INFINITY;
            st[2][tid] = ok ? stv[2] : 0.f;
        }
    };

    // one query block: compute from (qs, os, st) while the next block streams
    // into (qn, on, sn).  Only the diagonal block (qb == c) needs visibility
    // masks: it is the only block with keys past some row, and the only block
    // of the last column, whose keys may run past L.  Elsewhere every key is
    // visible to every row.
    auto block = [&](auto diag_tag, int qb, const uint8_t* qs, const uint8_t* os, const float (*st)[BQ],
                     uint8_t* qn, uint8_t* on, float (*sn)[BQ]) {
        constexpr bool diag = decltype(diag_tag)::value;
        const int r0 = qb * BQ;
        const bool more = qb + 1 < nqb;
        if (more) {
            stats_load(r0 + BQ);
            tile_async(q, qn, r0 + BQ);
            tile_async(dout, on, r0 + BQ);
        }
        // S (rows x keys) = Q K^T: 4 row blocks of 32, 8 k-steps
        f32x16 sacc[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(lds_ptr(lds_addr_of(qs) + 8192 * rb) + qoff[s]);
                sacc[rb] = mfma32(a, kf[s], sacc[rb]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        bool keep = tile_exists;
        if (GATED) {
            bool vote = false;
            if (tile_exists) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int rl = 32 * rb + 8 * g + 4 * hl;  // 4 consecutive rows
                        const f32x4 th = *reinterpret_cast<const f32x4*>(&st[0][rl]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const bool vis = !diag || (kvalid && key <= r0 + rl + x);
                            vote |= vis && sacc[rb][4 * g + x] >= th[x];
                        }
                    }
            }
            const bool wv = wave_any(vote);
            const int par = qb & 1;
            if (lane == 0) vote_sm[par][wave] = wv ? 1 : 0;
            lds_barrier();  // the next block's prefetch stays in flight
            const int pair = wave >> 1;
            keep = tile_exists && (vote_sm[par][2 * pair] | vote_sm[par][2 * pair + 1]) != 0;
        }
        if (aux_bits && keep && (wave & 1) == 0 && lane == 0)
            atomicOr(&aux_bits[(long(bh) * nqb + qb) * words + (tw >> 5)], 1u << (tw & 31));
        if (keep) {
            // P = exp(s - lse) (zero where invisible; lse2 = +inf on rows past L),
            // kept only as bf16 B operands: step (rb, hf) holds rows
            // 32rb + 16hf + 8(e/4) + 4hl + e%4 of this lane's key.
            u32x4 pf[4][2];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int rl = 32 * rb + 8 * g + 4 * hl;
                    const f32x4 lz = *reinterpret_cast<const f32x4*>(&st[1][rl]);
                    float p[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        // keys past L only reach their own (unstored) dK/dV rows: no mask needed
                        const bool vis = !diag || key <= r0 + rl + x;
                        p[x] = vis ? fast_exp2(fmaf(sacc[rb][4 * g + x], scale_log2, -lz[x])) : 0.f;
                    }
                    pf[rb][g >> 1][2 * (g & 1)] = pack_bf16x2(p[0], p[1]);
                    pf[rb][g >> 1][2 * (g & 1) + 1] = pack_bf16x2(p[2], p[3]);
                }
            __builtin_amdgcn_sched_barrier(0);
            // dV^T (d x keys) += dO^T P : A = dO^T (transposed read), B = P (lane = key)
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const u32x4 a = tr_operand_at(lds_addr_of(os) + 256 * (32 * rb + 16 * hf), troff[db]);
                        dvacc[db] = mfma32(a, pf[rb][hf], dvacc[db]);
                    }
            __builtin_amdgcn_sched_barrier(0);
            // dP (rows x keys) = dO V^T ; dS = P (dP - D), P taken from its bf16 operand copy
            u32x4 dsf[4][2];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                f32x16 pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(lds_ptr(lds_addr_of(os) + 8192 * rb) + qoff[s]);
                    pacc = mfma32(a, vf[s], pacc);
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 dd = *reinterpret_cast<const f32x4*>(&st[2][32 * rb + 8 * g + 4 * hl]);
                    const uint32_t w0 = pf[rb][g >> 1][2 * (g & 1)], w1 = pf[rb][g >> 1][2 * (g & 1) + 1];
                    const float p0 = __uint_as_float(w0 << 16), p1 = __uint_as_float(w0 & 0xffff0000u);
                    const float p2 = __uint_as_float(w1 << 16), p3 = __uint_as_float(w1 & 0xffff0000u);
                    dsf[rb][g >> 1][2 * (g & 1)] =
                        pack_bf16x2(p0 * (pacc[4 * g + 0] - dd[0]), p1 * (pacc[4 * g + 1] - dd[1]));
                    dsf[rb][g >> 1][2 * (g & 1) + 1] =
                        pack_bf16x2(p2 * (pacc[4 * g + 2] - dd[2]), p3 * (pacc[4 * g + 3] - dd[3]));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // dK^T (d x keys) += Q^T dS
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const u32x4 a = tr_operand_at(lds_addr_of(qs) + 256 * (32 * rb + 16 * hf), troff[db]);
                        dkacc[db] = mfma32(a, dsf[rb][hf], dkacc[db]);
                    }
        }
        if (more) stats_store(sn);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's loads into the next buffer landed
        lds_barrier();                       // next buffer complete; every wave is done with this one
    };

    // prologue: first block into buffer A
    tile_async(q, qsA, c * BQ);
    tile_async(dout, osA, c * BQ);
    stats_load(c * BQ);
    stats_store(stA);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    lds_barrier();
    // diagonal block from buffer A, then pairs of blocks B->A, A->B with static buffers
    block(std::true_type{}, c, qsA, osA, stA, qsB, osB, stB);
    for (int qb = c + 1; qb < nqb; qb += 2) {
        block(std::false_type{}, qb, qsB, osB, stB, qsA, osA, stA);
        if (qb + 1 < nqb) block(std::false_type{}, qb + 1, qsA, osA, stA, qsB, osB, stB);
    }

    // accumulators hold dK^T, dV^T: lane = key, register r of block db = d 32db + 8(r/4) + 4hl + r%4
    if (kvalid) {
        bf16_t* krow = dk + hoff + long(key) * D;
        bf16_t* vrow = dv + hoff + long(key) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 wk, wv;
                wk[0] = pack_bf16x2(dkacc[db][4 * g + 0] * scale, dkacc[db][4 * g + 1] * scale);
                wk[1] = pack_bf16x2(dkacc[db][4 * g + 2] * scale, dkacc[db][4 * g + 3] * scale);
                wv[0] = pack_bf16x2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
                wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                *reinterpret_cast<u32x2*>(krow + 32 * db + 8 * g + 4 * hl) = wk;
                *reinterpret_cast<u32x2*>(vrow + 32 * db + 8 * g + 4 * hl) = wv;
            }
    }
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
    const int BH = a.B * a.H;
    const int ncol = (a.L + 127) / 128;
    dim3 g1(unsigned(ncol) * unsigned(BH)), g2(unsigned(a.nqb) * unsigned(BH)), blk(256);
    const bool st = a.kept || a.legal || a.bits;
    hipError_t e = mark(a.ev[1], s);
    if (e != hipSuccess) return e;
    if (a.gated)
        hipLaunchKernelGGL((bwd_dkdv_bf16_d128<true>), g1, blk, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,
                           (const bf16_t*)a.v, (const bf16_t*)a.dout, a.Dv, a.lse2, a.thr, (bf16_t*)a.dk,
                           (bf16_t*)a.dv, BH, a.L, a.nqb, ncol, a.words, a.scale, a.scale_log2, a.aux_bits);
    else
        hipLaunchKernelGGL((bwd_dkdv_bf16_d128<false>), g1, blk, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,
                           (const bf16_t*)a.v, (const bf16_t*)a.dout, a.Dv, a.lse2, a.thr, (bf16_t*)a.dk,
                           (bf16_t*)a.dv, BH, a.L, a.nqb, ncol, a.words, a.scale, a.scale_log2, a.aux_bits);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(a.ev[2], s);
    if (e != hipSuccess) return e;
#define MALA_DQ_LAUNCH(G, S)                                                                                  \
    hipLaunchKernelGGL((bwd_dq_bf16_d128<G, S>), g2, blk, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,       \
                       (const bf16_t*)a.v, (const bf16_t*)a.dout, a.Dv, a.lse2, a.thr, (bf16_t*)a.dq, BH, a.L, \
                       a.nqb, a.words, a.scale, a.scale_log2, a.kept, a.legal, a.bits)
    if (a.gated) {
        if (st) MALA_DQ_LAUNCH(true, true);
        else MALA_DQ_LAUNCH(true, false);
    } else {
        if (st) MALA_DQ_LAUNCH(false, true);
        else MALA_DQ_LAUNCH(false, false);
    }
#undef MALA_DQ_LAUNCH
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(a.ev[3], s);
    return e;
}

}  // namespace mala
