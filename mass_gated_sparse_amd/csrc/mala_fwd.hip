// MALA forward, bf16 inputs, head dim 128, 128x64 tiles, on gfx950 MFMA.
//
// Source: "MassAlloc Attention: Let Attention Allocate Its Own Compute"
// (agihunt.info digest).  Threshold paragraph: after each QK tile the largest
// per-key contribution ratio of a row is compared with tau/Lq.  Forward
// paragraph: the ratio uses the running online-softmax normalizer, the tile is
// kept for the whole query block if any row keeps it, tiles are visited from
// the diagonal toward earlier keys, the first legal tile is always kept, and
// the final log-normalizer is written.  Savings paragraph: a skipped tile loads
// no V and does no softmax update or PV.
//
// Work decomposition.  One workgroup (4 waves) owns one 128-row query block =
// one vote block.  Wave w owns rows 32w..32w+31.  Scores are computed
// transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS,
// B = Q held in registers): lane l then holds query row l%32 and 16 keys per
// 32-key block, so every per-row operation (test, max, exp, rescale) is
// lane-local and the whole test is one compare per score plus a wave ballot
// and a 4-way OR through LDS.  The output is kept transposed as well,
// O^T += V^T P^T: P^T comes straight from the score registers (as bf16) and
// V^T is read from the row-major V tile with transposing LDS reads.
//
// Pipeline.  Tiles flow through three overlapped stages.  While tile t is
// tested, the scores of tile t-1 are computed and the PV product of tile t+1
// is accumulated:
//   * K tiles arrive by direct global->LDS loads one tile ahead (two slots);
//   * the running statistics (m, l) of a kept tile are updated right after its
//     vote -- they need no V -- so the next vote never waits for V;
//   * V of a kept tile is requested right after its vote and consumed one
//     iteration later: O += P_{t+1} V_{t+1} (in the frame of m after tile t+1),
//     then O *= exp2(m_{t+1} - m_t).  This is the same recurrence as the
//     undelayed update, applied in the same order.
// Per iteration: one barrier (vote exchange, next K visible), plus one when
// the previous tile was kept (its V visible).
// The test runs in the raw dot-product domain: with c = scale*log2(e) and the
// running state kept as m2 = max s*log2(e) and l, row i keeps the tile iff
// max_j <q_i,k_j> >= (m2 + log2 l + log2 tau - log2 Lq_i) / c,
// i.e. exp(max_j s_ij - m)/l >= tau/Lq_i.  An empty row (l = 0) keeps.
#include <float.h>

#include <type_traits>

#include "mala_kernels.hpp"

namespace mala {

namespace fwdk {
constexpr int BQ = 128, BK = 64, D = 128;
}  // namespace fwdk

template <bool GATED, bool STATS>
__global__ __launch_bounds__(256, 2) void fwd_bf16_d128(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                        const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                                        float* __restrict__ lse, int BH, int G, int L, int P, int Lk,
                                                        int Lkcap, int nqb, int words,
                                                        float scale_log2, float log2_tau, int32_t* __restrict__ kept,
                                                        int32_t* __restrict__ legal, uint32_t* __restrict__ bits,
                                                        float* __restrict__ tstat) {
    using namespace fwdk;
    __shared__ __attribute__((aligned(1024))) uint8_t kslot[2][BK * 256];  // K tile t in kslot[t & 1]
    __shared__ __attribute__((aligned(1024))) uint8_t vslot[2][BK * 256];  // V tile t in vslot[t & 1]
    __shared__ int vote_sm[2][4];
    __shared__ float tstat_sm[2][4];  // statistics only: each wave's largest test margin

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    int qrank, bh;
    balanced_item(int(blockIdx.x), BH, max(1, nqb / 8), qrank, bh);
    const int qb = nqb - 1 - qrank;  // longest query blocks first
    const long hoff = long(bh) * L * D;              // this query head
    const long kvoff = long(bh / G) * Lkcap * D;     // its KV head (G query heads per KV head)
    const bf16_t* kh = k + kvoff;
    const bf16_t* vh = v + kvoff;
    const int row = qb * BQ + wave * 32 + j;
    const bool rvalid = row < L;

    // Q as the B operand of S^T = K Q^T: step s holds q[row][16s + 8hl .. +8].
    // Rows past L read row L-1; they never vote and are never stored.
    u32x4 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qf[s] = *reinterpret_cast<const u32x4*>(q + hoff + long(min(row, L - 1)) * D + 16 * s + 8 * hl);

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;
    const float log2_lq = fast_log2(float(P + row + 1));  // the row sits at key position P + row
    const float inv_scale_log2 = 1.f / scale_log2;
    const int jmax = (P + min(qb * BQ + BQ, L) - 1) / BK;
    const int tdiag = (P + qb * BQ) / BK;  // tiles t >= tdiag reach the block's first row
    const int ntk = (Lk + BK - 1) / BK;    // key tiles of the cache (test-statistic row length)

    auto tile_dma = [&](const bf16_t* g, uint8_t* dst, int t) {
        const uint32_t la = lds_addr_of(dst) + 4096 * wave;
        const int rmax = Lk - 1 - t * BK;  // keys past Lk read key Lk-1 (masked)
        const bf16_t* gt = g + long(t) * BK * D;  // wave-uniform
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = 16 * wave + 4 * it + (lane >> 4);
            const uint32_t off = uint32_t(min(r, rmax) * D + (((lane & 15) ^ rowkey(r)) << 3)) * 2u;
            dma16s(gt, off, __builtin_amdgcn_readfirstlane(la + 1024 * it));
        }
    };
    int koff[8];  // K operand of step s: row j, chunk 2s + hl
#pragma unroll
    for (int s = 0; s < 8; ++s) koff[s] = swz(j, 2 * s + hl);
    int voff[4][2];
    tr_offsets(lane, voff);
    // The 16 products run from a register ring: the K operand of product i
    // (key block i & 1, step i >> 1) is read three products ahead, with a
    // scheduling fence after each product so that the reads stay ahead.
    auto scores = [&](const uint8_t* kt, f32x16* sacc) {
        const uint32_t kb0 = lds_addr_of(kt);
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
    // O^T (d x rows) += V^T (d x keys) P^T (keys x rows)
    // product i = (db = i / 4, kb = (i / 2) % 2, hf = i % 2), its transposed
    // V operand read three products ahead (ring, fenced as above)
    auto pv = [&](const uint8_t* vt, const u32x4 (*pf)[2]) {
        const uint32_t vb = lds_addr_of(vt);
        auto rd = [&](int i) -> u32x4 {
            return tr_operand_at(vb + 256 * (32 * ((i >> 1) & 1) + 16 * (i & 1)), voff[i >> 2]);
        };
        u32x4 ring[4];
#pragma unroll
        for (int i = 0; i < 3; ++i) ring[i] = rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 3 < 16) ring[(i + 3) & 3] = rd(i + 3);
            __builtin_amdgcn_sched_barrier(0);
            oacc[i >> 2] = mfma32(ring[i & 3], pf[(i >> 1) & 1][i & 1], oacc[i >> 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    int nkept = 0;
    uint32_t word = 0;
    if (STATS && bits && tid == 0)
        for (int w = (jmax >> 5) + 1; w < words; ++w) bits[(long(bh) * nqb + qb) * words + w] = 0u;

    // prologue: K(jmax) and K(jmax-1) visible; scores of tile jmax; then
    // K(jmax-2) requested into the slot K(jmax) used
    tile_dma(kh, kslot[jmax & 1], jmax);
    if (jmax >= 1) tile_dma(kh, kslot[(jmax - 1) & 1], jmax - 1);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    lds_barrier();
    f32x16 sc[2], sn[2];  // scores of the tile being tested / of the next tile
    scores(kslot[jmax & 1], sc);
    if (jmax >= 2) {
        lds_barrier();  // every wave is done with K(jmax)
        tile_dma(kh, kslot[jmax & 1], jmax - 2);
    }

    u32x4 ppend[2][2];  // P of the previous kept tile (bf16), waiting for its V
    bool pend = false;  // previous tile kept (its V in flight)
    // Per tile t, one barrier.  Before it: the vote of t and the scores of t-1
    // (K(t-1) has been visible since the previous barrier), so the MFMAs hide
    // the vote exchange.  After it: the K(t-3) and V(t) requests (each has a
    // whole step to land), this tile's statistics, the PV of the previous kept
    // tile t+1 and this tile's rescale.
    // One step per tile; the tile parity PAR = t & 1 is a compile-time constant,
    // so every LDS slot address is a constant (it folds into the instructions'
    // offset fields) and the score registers are renamed, not copied.
    auto step = [&](auto par_tag, int t) {
        constexpr int PAR = decltype(par_tag)::value;
        // causal mask on the tiles that reach the diagonal: register r of key
        // block kb holds key t*64 + 32kb + 8(r/4) + 4hl + r%4, invisible when > row
        if (t >= tdiag) {
            const int lim = P + row - t * BK - 4 * hl;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = -INFINITY;
        }
        // ---- test + block vote
        // lane-local row maximum: the vote needs it, a kept tile's statistics too
        float mx = sc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        if (GATED) {
            float thr_raw;
            if (!rvalid) thr_raw = INFINITY;           // padding rows never vote
            else if (lsum == 0.f) thr_raw = -FLT_MAX;  // empty row: any visible key keeps
            else thr_raw = (m2 + fast_log2(lsum) + log2_tau - log2_lq) * inv_scale_log2;
            const bool wv = wave_any(mx >= thr_raw);
            if (lane == 0) vote_sm[PAR][wave] = wv ? 1 : 0;
            if (STATS && tstat) {
                // log2 of the tile's test statistic: the largest margin
                // c*max_j s_ij - (m2 + log2 l + log2 tau - log2 Lq) of a voting row
                // (+inf for an empty state; rows without a visible key abstain)
                const float rmx = fmaxf(mx, shfl_xor_f(mx, 32));
                float dl;
                if (!rvalid || rmx == -INFINITY) dl = -INFINITY;
                else if (lsum == 0.f) dl = INFINITY;
                else dl = rmx * scale_log2 - (m2 + fast_log2(lsum) + log2_tau - log2_lq);
#pragma unroll
                for (int m = 16; m >= 1; m >>= 1) dl = fmaxf(dl, shfl_xor_f(dl, m));
                if (lane == 0) tstat_sm[PAR][wave] = dl;
            }
        }
        if (t >= 1) scores(kslot[1 - PAR], sn);
        // K(t-2) and V(t+1), requested in the previous step, have landed (with
        // statistics on, thread 0 also waits for its keep-bit stores)
        __builtin_amdgcn_s_waitcnt(0x0f70);
        lds_barrier();  // votes, K(t-2), V(t+1) visible; every wave is done with kslot[1 - PAR]
        int vflags = 1;
        if (GATED) vflags = vote_sm[PAR][0] | vote_sm[PAR][1] | vote_sm[PAR][2] | vote_sm[PAR][3];
        const bool keep = vflags != 0;
        if (STATS && tstat && tid == 0)  // tau = 0 runs no test: NaN
            tstat[(long(bh) * nqb + qb) * ntk + t] =
                GATED ? fmaxf(fmaxf(tstat_sm[PAR][0], tstat_sm[PAR][1]), fmaxf(tstat_sm[PAR][2], tstat_sm[PAR][3]))
                      : NAN;
        if (t >= 3) tile_dma(kh, kslot[1 - PAR], t - 3);  // K(t-3) into the slot K(t-1) used
        if (keep) tile_dma(vh, vslot[PAR], t);              // V only for kept tiles

        float alpha = 1.f;
        if (keep) {
            // statistics (no V needed); P_t = exp2(s*c - m) kept in place
            mx = max_halves(mx);
            const float mn = fmaxf(m2, mx * scale_log2);
            const float mref = (mn == -INFINITY) ? 0.f : mn;
            float lpart = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sc[kb][r], scale_log2, -mref));
                    sc[kb][r] = p;
                    lpart += p;
                }
            lpart = sum_halves(lpart);
            alpha = fast_exp2(m2 - mref);
            lsum = lsum * alpha + lpart;
            m2 = mn;
        }
        // PV of the previous kept tile (in its own frame), then this tile's rescale
        if (pend) pv(vslot[1 - PAR], ppend);
        if (keep) {
            if (__ballot(alpha != 1.f) != 0ull) {  // skipped when no row's max moved (exact)
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            // P^T as B operands: step (kb, hf) holds score registers 8*hf .. 8*hf+7
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ppend[kb][hf][e] = pack_bf16x2(sc[kb][8 * hf + 2 * e], sc[kb][8 * hf + 2 * e + 1]);
        }
        pend = keep;

        if (STATS && tid == 0) {
            nkept += keep;
            if (keep) word |= 1u << (t & 31);
            if (bits && (t & 31) == 0) {
                bits[(long(bh) * nqb + qb) * words + (t >> 5)] = word;
                word = 0;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[kb] = sn[kb];
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    int t = jmax;
    if (t & 1) step(Odd{}, t--);
    for (; t >= 0; t -= 2) {
        step(Even{}, t);
        if (t >= 2) step(Odd{}, t - 1);
    }
    if (pend) {  // PV of the last kept tile (tile 0)
        __builtin_amdgcn_s_waitcnt(0x0f70);
        lds_barrier();
        pv(vslot[0], ppend);
    }

    // ---- epilogue: O = acc / l (bf16), lse = ln(sum) in natural log
    if (rvalid) {
        const float inv = 1.f / lsum;
        bf16_t* orow = o + hoff + long(row) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hl) = w;
            }
        if (hl == 0) lse[long(bh) * L + row] = (m2 + fast_log2(lsum)) * kLn2;
    }
    if (STATS && tid == 0) {
        if (kept) kept[long(bh) * nqb + qb] = nkept;
        if (legal) legal[long(bh) * nqb + qb] = jmax + 1;
    }
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
    const int BH = a.B * a.H;
    if (a.Hkv < 1 || a.H % a.Hkv) return hipErrorInvalidValue;  // the API checked this already
    dim3 grid(unsigned(a.nqb) * unsigned(BH)), block(256);
    const bool st = a.kept || a.legal || a.bits || a.tstat;
#define MALA_FWD_LAUNCH(GT, ST)                                                                           \
    hipLaunchKernelGGL((fwd_bf16_d128<GT, ST>), grid, block, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,   \
                       (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, BH, a.H / a.Hkv, a.L, a.P, a.Lk, a.Lkcap,  \
                       a.nqb, a.words,                                                                       \
                       a.scale_log2, a.log2_tau, a.kept, a.legal, a.bits, a.tstat)
    // tau = 0 without statistics runs the gated kernel too: its thresholds
    // are -inf (log2 0), so every legal tile is kept and the results are the
    // ungated kernel's bit for bit, and it measured faster (17.06 against
    // 17.39 ms at 128K, 2.02 against 2.06 ms at 32K); tau = 0 with statistics
    // keeps the ungated kernel, which forms no test statistic (NaN)
    if (a.gated || !st) {
        if (st) MALA_FWD_LAUNCH(true, true);
        else MALA_FWD_LAUNCH(true, false);
    } else {
        MALA_FWD_LAUNCH(false, true);
    }
#undef MALA_FWD_LAUNCH
    return hipGetLastError();
}

}  // namespace mala
