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
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane l then holds
// query row l%32 and 16 keys per 32-key block, so every per-row operation
// (test, max, exp, rescale) is lane-local and the whole test is one compare
// per score plus a wave ballot and a 4-way OR through LDS.  The output is also
// kept transposed, O^T += V^T P^T, so the online-softmax rescale stays
// lane-local; P^T comes straight from the score registers (converted to bf16)
// and V is written transposed into LDS when (and only when) a tile is kept.
//
// The test runs in the raw dot-product domain: with c = scale*log2(e) and the
// running state kept as m2 = max s*log2(e) and l, row i keeps the tile iff
// max_j <q_i,k_j> >= (m2 + log2 l + log2 tau - log2 Lq_i) / c,
// i.e. exp(max_j s_ij - m)/l >= tau/Lq_i.  An empty row (l = 0) keeps.
//
// LDS: K tile 64x128 bf16 (16 KiB, 16-byte chunks XOR-swizzled by key so the
// 32-key MFMA operand reads are conflict-free), V^T 128x64 bf16 with rows
// padded to 136 B (17 KiB).  The next K tile is prefetched into registers
// while the current one is scored.
#include <float.h>

#include "mala_kernels.hpp"

namespace mala {

namespace fwdk {
constexpr int BQ = 128, BK = 64, D = 128;
constexpr int VT = 136;  // bytes per V^T row in LDS
__device__ __forceinline__ int kswz(int key, int chunk) { return key * 256 + ((chunk ^ (key & 15)) << 4); }
}  // namespace fwdk

template <bool GATED, bool STATS>
__global__ __launch_bounds__(256, 2) void fwd_bf16_d128(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                        const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                                        float* __restrict__ lse, int BH, int L, int nqb, int words,
                                                        float scale_log2, float log2_tau, int32_t* __restrict__ kept,
                                                        int32_t* __restrict__ legal, uint32_t* __restrict__ bits) {
    using namespace fwdk;
    __shared__ __attribute__((aligned(16))) uint8_t ksm[BK * 256];
    __shared__ __attribute__((aligned(16))) uint8_t vsm[D * VT];
    __shared__ int vote_sm[4];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, j = lane & 31;
    const int qb = nqb - 1 - int(blockIdx.x) / BH;  // longest query blocks first
    const int bh = int(blockIdx.x) % BH;
    const long hoff = long(bh) * L * D;
    const bf16_t* qh = q + hoff;
    const bf16_t* kh = k + hoff;
    const bf16_t* vh = v + hoff;
    const int row = qb * BQ + wave * 32 + j;
    const bool rvalid = row < L;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const u32x2 z2 = {0u, 0u};

    // Q as the B operand of S^T = K Q^T: step s holds q[row][16s + 8hl .. +8].
    u32x4 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qf[s] = rvalid ? *reinterpret_cast<const u32x4*>(qh + long(row) * D + 16 * s + 8 * hl) : z4;

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;
    const float log2_lq = fast_log2(float(row + 1));
    const int jmax = (min(qb * BQ + BQ, L) - 1) / BK;

    // K tile loader: thread loads keys it*16 + tid/16 (it = 0..3), chunk tid%16.
    u32x4 kreg[4];
    auto load_k = [&](int t) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int jg = t * BK + it * 16 + (tid >> 4);
            kreg[it] = (jg < L) ? *reinterpret_cast<const u32x4*>(kh + long(jg) * D + (tid & 15) * 8) : z4;
        }
    };
    auto store_k = [&]() {
#pragma unroll
        for (int it = 0; it < 4; ++it)
            *reinterpret_cast<u32x4*>(ksm + kswz(it * 16 + (tid >> 4), tid & 15)) = kreg[it];
    };

    int nkept = 0;
    uint32_t word = 0;
    if (STATS && bits && tid == 0)
        for (int w = (jmax >> 5) + 1; w < words; ++w) bits[(long(bh) * nqb + qb) * words + w] = 0u;

    load_k(jmax);
    store_k();
    __syncthreads();

    for (int t = jmax; t >= 0; --t) {
        if (t > 0) load_k(t - 1);  // prefetch the next tile while this one is scored

        // ---- scores S^T (keys x rows) of tile t: 2 blocks of 32 keys, 8 k-steps over d
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(ksm + kswz(32 * kb + j, 2 * s + hl));
                sacc[kb] = mfma32(a, qf[s], sacc[kb]);
            }
        }
        // causal mask on the tiles that reach the diagonal (key > row invisible)
        if (t >= 2 * qb) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t * BK + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (key > row) sacc[kb][r] = -INFINITY;
                }
        }

        // ---- test + block vote
        bool keep = true;
        if (GATED) {
            float thr_raw;
            if (!rvalid) thr_raw = INFINITY;               // padding rows never vote
            else if (lsum == 0.f) thr_raw = -FLT_MAX;      // empty row: any visible key keeps
            else thr_raw = (m2 + fast_log2(lsum) + log2_tau - log2_lq) / scale_log2;
            bool vote = false;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) vote |= sacc[kb][r] >= thr_raw;
            const bool wv = wave_any(vote);
            if (lane == 0) vote_sm[wave] = wv ? 1 : 0;
            __syncthreads();  // votes visible; all waves are done reading this K tile
            keep = (vote_sm[0] | vote_sm[1] | vote_sm[2] | vote_sm[3]) != 0;
        } else {
            __syncthreads();
        }

        if (keep) {
            // V tile loads (consumed after the softmax update below).
            // 16 units of 4 keys x 32 d; unit u = (2*wave + hl) + 8*it.
            u32x2 vr[2][4];
            int vdg[2], vkg[2];
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int u = (2 * wave + hl) + 8 * it;
                vdg[it] = 8 * (u & 3) + (j & 7);    // d = 4*vdg .. +3
                vkg[it] = 4 * (u >> 2) + (j >> 3);  // keys 4*vkg .. +3
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = t * BK + 4 * vkg[it] + i;
                    vr[it][i] = key < L ? *reinterpret_cast<const u32x2*>(vh + long(key) * D + 4 * vdg[it]) : z2;
                }
            }

            // online softmax update of this row (lane-local; the two lane halves share a row)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            const float mn = fmaxf(m2, mx * scale_log2);
            const float mref = (mn == -INFINITY) ? 0.f : mn;
            float lpart = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sacc[kb][r], scale_log2, -mref));
                    sacc[kb][r] = p;
                    lpart += p;
                }
            lpart += shfl_xor_f(lpart, 32);
            const float alpha = fast_exp2(m2 - mref);
            lsum = lsum * alpha + lpart;
            m2 = mn;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

            // P^T as B operands: step (kb, half) holds score registers 8*half .. 8*half+7
            u32x4 pf[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pf[kb][hf][e] = pack_bf16x2(sacc[kb][8 * hf + 2 * e], sacc[kb][8 * hf + 2 * e + 1]);

            // V -> V^T in LDS: 4x4 (key x d) blocks transposed in registers
#pragma unroll
            for (int it = 0; it < 2; ++it) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sh = (e & 1) * 16;
                    uint32_t x0, x1, x2, x3;
                    if (e < 2) { x0 = vr[it][0][0]; x1 = vr[it][1][0]; x2 = vr[it][2][0]; x3 = vr[it][3][0]; }
                    else       { x0 = vr[it][0][1]; x1 = vr[it][1][1]; x2 = vr[it][2][1]; x3 = vr[it][3][1]; }
                    u32x2 w;
                    w[0] = ((x0 >> sh) & 0xffffu) | (((x1 >> sh) & 0xffffu) << 16);
                    w[1] = ((x2 >> sh) & 0xffffu) | (((x3 >> sh) & 0xffffu) << 16);
                    *reinterpret_cast<u32x2*>(vsm + (4 * vdg[it] + e) * VT + 8 * vkg[it]) = w;
                }
            }
            __syncthreads();  // V^T ready

            // O^T (d x rows) += V^T (d x keys) P^T (keys x rows)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint8_t* vrow = vsm + (32 * db + j) * VT;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int key0 = 32 * kb + 16 * hf + 4 * hl;
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 2 * key0);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 2 * (key0 + 8));
                        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                        oacc[db] = mfma32(a, pf[kb][hf], oacc[db]);
                    }
            }
        }

        if (STATS && tid == 0) {
            nkept += keep;
            if (keep) word |= 1u << (t & 31);
            if (bits && (t & 31) == 0) {
                bits[(long(bh) * nqb + qb) * words + (t >> 5)] = word;
                word = 0;
            }
        }
        if (t > 0) store_k();
        __syncthreads();  // next K tile in LDS; V^T reads of this tile done
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
    dim3 grid(unsigned(a.nqb) * unsigned(BH)), block(256);
    const bool st = a.kept || a.legal || a.bits;
#define MALA_FWD_LAUNCH(G, S)                                                                                  \
    hipLaunchKernelGGL((fwd_bf16_d128<G, S>), grid, block, 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,       \
                       (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, BH, a.L, a.nqb, a.words, a.scale_log2, a.log2_tau, \
                       a.kept, a.legal, a.bits)
    if (a.gated) {
        if (st) MALA_FWD_LAUNCH(true, true);
        else MALA_FWD_LAUNCH(true, false);
    } else {
        if (st) MALA_FWD_LAUNCH(false, true);
        else MALA_FWD_LAUNCH(false, false);
    }
#undef MALA_FWD_LAUNCH
    return hipGetLastError();
}

}  // namespace mala
