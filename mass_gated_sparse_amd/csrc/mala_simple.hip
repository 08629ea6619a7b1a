// Scalar (non-MFMA) MALA kernels for fp32 inputs with d = 64 and 64x64 tiles.
//
// One thread per query row (forward, dQ) or per key (dK/dV).  These carry the
// fp32 instantiation of the operator; the bf16 d = 128 instantiation lives in
// the MFMA kernels.  Source: "MassAlloc Attention: Let Attention Allocate Its
// Own Compute" (agihunt.info digest) -- threshold, forward and backward
// paragraphs.  All tests are done in the log2 domain: with s2 = s * log2(e)
// a row keeps a tile iff max_j s2_ij >= m2_i + log2(l_i) + log2(tau) - log2(Lq_i),
// which is the ratio test exp(max s - m)/l >= tau/Lq written with logarithms.
#include <float.h>

#include "mala_kernels.hpp"

namespace mala {

// --------------------------------------------------------------------- forward
template <int BQ, int BK, int D, bool GATED>
__global__ __launch_bounds__(BQ) void simple_fwd_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ v, float* __restrict__ o,
                                                     float* __restrict__ lse, int L, int nqb, float scale_log2,
                                                     float log2_tau, int32_t* kept, int32_t* legal,
                                                     uint32_t* bits, int words) {
    __shared__ float ks[BK][D];
    __shared__ float vs[BK][D];
    __shared__ float ss[BQ][BK + 1];
    const int tid = threadIdx.x;
    const int qb = nqb - 1 - int(blockIdx.x);  // longest blocks first
    const long bh = blockIdx.y;
    const float* qh = q + bh * long(L) * D;
    const float* kh = k + bh * long(L) * D;
    const float* vh = v + bh * long(L) * D;
    const int row = qb * BQ + tid;
    const bool valid = row < L;

    float qr[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = valid ? qh[long(row) * D + c] : 0.f;
        acc[c] = 0.f;
    }
    float m2 = -INFINITY, l = 0.f;
    const float log2_lq = fast_log2(float(row + 1));
    const int rlast = min(qb * BQ + BQ, L) - 1;
    const int jmax = rlast / BK;
    int nkept = 0;
    uint32_t word = 0;
    if (bits && tid == 0)
        for (int w = (jmax >> 5) + 1; w < words; ++w) bits[(bh * nqb + qb) * long(words) + w] = 0u;

    for (int t = jmax; t >= 0; --t) {
        const int c0 = t * BK;
        __syncthreads();
        for (int e = tid; e < BK * D; e += BQ) {
            const int jj = e / D, c = e % D;
            ks[jj][c] = (c0 + jj < L) ? kh[long(c0 + jj) * D + c] : 0.f;
        }
        __syncthreads();
        float smax = -INFINITY;
        for (int jj = 0; jj < BK; ++jj) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot = fmaf(qr[c], ks[jj][c], dot);
            const float s2 = (valid && c0 + jj <= row) ? dot * scale_log2 : -INFINITY;
            ss[tid][jj] = s2;
            smax = fmaxf(smax, s2);
        }
        bool keep = true;
        if (GATED) {
            const bool vis = valid && c0 <= row;
            const bool vote = vis && (l == 0.f || smax >= m2 + fast_log2(l) + log2_tau - log2_lq);
            keep = __syncthreads_or(vote) != 0;
        }
        if (keep) {
            for (int e = tid; e < BK * D; e += BQ) {
                const int jj = e / D, c = e % D;
                vs[jj][c] = (c0 + jj < L) ? vh[long(c0 + jj) * D + c] : 0.f;
            }
            __syncthreads();
            if (valid && c0 <= row) {
                const float mn = fmaxf(m2, smax);
                const float a = fast_exp2(m2 - mn);
                l *= a;
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] *= a;
                for (int jj = 0; jj < BK; ++jj) {
                    const float p = fast_exp2(ss[tid][jj] - mn);  // -inf (invisible) gives 0
                    l += p;
#pragma unroll
                    for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[jj][c], acc[c]);
                }
                m2 = mn;
            }
        }
        if (tid == 0) {
            nkept += keep;
            if (keep) word |= 1u << (t & 31);
            if (bits && ((t & 31) == 0 || t == 0)) {
                bits[(bh * nqb + qb) * long(words) + (t >> 5)] = word;
                word = 0;
            }
        }
    }
    if (valid) {
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < D; ++c) o[bh * long(L) * D + long(row) * D + c] = acc[c] * inv;
        lse[bh * long(L) + row] = (m2 + fast_log2(l)) * kLn2;
    }
    if (tid == 0) {
        if (kept) kept[bh * nqb + qb] = nkept;
        if (legal) legal[bh * nqb + qb] = jmax + 1;
    }
}

// ------------------------------------------------------------------- backward
// Shared per-row backward state, computed once by bwd_prep:
//   Dv[i]   = sum_c dO_ic O_ic
//   lse2[i] = lse_i * log2(e)
//   thr[i]  = (lse2_i + log2(tau) - log2(i+1)) / (scale*log2(e))  -- the raw
//             dot-product level a score must reach for row i to keep a tile.
// Both backward kernels read these same values, so their decisions agree.
// Row 0 is exact: it sees only key 0, which the forward always keeps, so its
// final normalizer is exp(s_00), P_00 = 1 and its vote is 1 >= tau (equality
// keeps).  A threshold derived from the fp32 lse would leave that tie at
// tau = 1 to rounding, so row 0 gets -FLT_MAX (its one finite score always
// passes; masked scores, -inf, never do) when tau <= 1 and +inf otherwise.
__device__ __forceinline__ float bwd_row_threshold(int i, float l2, float log2_tau, float scale_log2) {
    if (i == 0) return log2_tau <= 0.f ? -FLT_MAX : INFINITY;
    return (l2 + log2_tau - fast_log2(float(i + 1))) / scale_log2;
}
template <typename T, int D>
__global__ void bwd_prep(const T* __restrict__ o, const T* __restrict__ dout, const float* __restrict__ lse,
                         float* __restrict__ Dv, float* __restrict__ lse2, float* __restrict__ thr, long rows, int L,
                         float scale_log2, float log2_tau) {
    const long r = long(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    if (r >= rows) return;
    float s = 0.f;
    for (int c = lane; c < D; c += 64) s += to_f32(o[r * D + c]) * to_f32(dout[r * D + c]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) {
        const int i = int(r % L);
        const float l2 = lse[r] * kLog2e;
        Dv[r] = s;
        lse2[r] = l2;
        thr[r] = bwd_row_threshold(i, l2, log2_tau, scale_log2);
    }
}

// The same per-row state for bf16 rows of 128: 16 lanes per row, each
// reading 16 bytes of O and of dO (one wave covers four rows).
__global__ __launch_bounds__(256) void bwd_prep_bf16_d128(const bf16_t* __restrict__ o,
                                                          const bf16_t* __restrict__ dout,
                                                          const float* __restrict__ lse, float* __restrict__ Dv,
                                                          float* __restrict__ lse2, float* __restrict__ thr,
                                                          long rows, int L, float scale_log2, float log2_tau) {
    constexpr int D = 128;
    const long r = (long(blockIdx.x) * 256 + threadIdx.x) >> 4;
    const int sub = threadIdx.x & 15;
    float s = 0.f;
    if (r < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + r * D + 8 * sub);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dout + r * D + 8 * sub);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), s);
            s = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), s);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);  // within the row's 16 lanes
    if (r < rows && sub == 0) {
        const int i = int(r % L);
        const float l2 = lse[r] * kLog2e;
        Dv[r] = s;
        lse2[r] = l2;
        thr[r] = bwd_row_threshold(i, l2, log2_tau, scale_log2);
    }
}

// dK, dV: one thread per key of a BK-key tile column; loops over query blocks.
template <int BQ, int BK, int D, bool GATED>
__global__ __launch_bounds__(BK, 1) void simple_bwd_dkdv_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    const float* __restrict__ thr, float* __restrict__ dk, float* __restrict__ dv, int L, int nqb, int ntiles,
    float scale, float scale_log2, uint32_t* aux_bits, int words) {
    __shared__ float qs[BQ][D];
    __shared__ float ds_[BQ][D];
    __shared__ float rstat[3][BQ];
    const int tid = threadIdx.x;
    const int t = ntiles - 1 - int(blockIdx.x);
    const long bh = blockIdx.y;
    const long base = bh * long(L) * D;
    const int j = t * BK + tid;
    const bool kvalid = j < L;
    float kj[D], vj[D], gk[D], gv[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        kj[c] = kvalid ? k[base + long(j) * D + c] : 0.f;
        vj[c] = kvalid ? v[base + long(j) * D + c] : 0.f;
        gk[c] = 0.f;
        gv[c] = 0.f;
    }
    for (int qb = (t * BK) / BQ; qb < nqb; ++qb) {
        const int r0 = qb * BQ;
        __syncthreads();
        for (int e = tid; e < BQ * D; e += BK) {
            const int ii = e / D, c = e % D;
            const bool ok = r0 + ii < L;
            qs[ii][c] = ok ? q[base + long(r0 + ii) * D + c] : 0.f;
            ds_[ii][c] = ok ? dout[base + long(r0 + ii) * D + c] : 0.f;
        }
        for (int ii = tid; ii < BQ; ii += BK) {
            const bool ok = r0 + ii < L;
            rstat[0][ii] = ok ? Dv[bh * L + r0 + ii] : 0.f;
            rstat[1][ii] = ok ? lse2[bh * L + r0 + ii] : 0.f;
            rstat[2][ii] = ok ? thr[bh * L + r0 + ii] : INFINITY;
        }
        __syncthreads();
        bool keep = true;
        if (GATED) {
            bool vote = false;
            for (int ii = 0; ii < BQ; ++ii) {
                const int i = r0 + ii;
                if (!kvalid || j > i || i >= L) continue;
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < D; ++c) dot = fmaf(qs[ii][c], kj[c], dot);
                vote |= dot >= rstat[2][ii];
            }
            keep = __syncthreads_or(vote) != 0;
        }
        if (aux_bits && tid == 0 && keep)
            atomicOr(&aux_bits[(bh * nqb + qb) * long(words) + (t >> 5)], 1u << (t & 31));
        if (!keep) continue;
        for (int ii = 0; ii < BQ; ++ii) {
            const int i = r0 + ii;
            if (!kvalid || j > i || i >= L) continue;
            float dot = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                dot = fmaf(qs[ii][c], kj[c], dot);
                dp = fmaf(ds_[ii][c], vj[c], dp);
            }
            const float p = fast_exp2(dot * scale_log2 - rstat[1][ii]);
            const float dsv = p * (dp - rstat[0][ii]) * scale;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                gv[c] = fmaf(p, ds_[ii][c], gv[c]);
                gk[c] = fmaf(dsv, qs[ii][c], gk[c]);
            }
        }
    }
    if (kvalid) {
#pragma unroll
        for (int c = 0; c < D; ++c) {
            dk[base + long(j) * D + c] = gk[c];
            dv[base + long(j) * D + c] = gv[c];
        }
    }
}

// dQ: one thread per query row; loops over the block's legal key tiles.
template <int BQ, int BK, int D, bool GATED>
__global__ __launch_bounds__(BQ, 1) void simple_bwd_dq_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ Dv, const float* __restrict__ lse2,
    const float* __restrict__ thr, float* __restrict__ dq, int L, int nqb, float scale, float scale_log2,
    int32_t* kept, int32_t* legal, uint32_t* bits, int words) {
    __shared__ float ks[BK][D];
    __shared__ float vs[BK][D];
    const int tid = threadIdx.x;
    const int qb = nqb - 1 - int(blockIdx.x);
    const long bh = blockIdx.y;
    const long base = bh * long(L) * D;
    const int row = qb * BQ + tid;
    const bool valid = row < L;
    float qr[D], dr[D], g[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = valid ? q[base + long(row) * D + c] : 0.f;
        dr[c] = valid ? dout[base + long(row) * D + c] : 0.f;
        g[c] = 0.f;
    }
    const float Di = valid ? Dv[bh * L + row] : 0.f;
    const float l2 = valid ? lse2[bh * L + row] : 0.f;
    const float th = valid ? thr[bh * L + row] : INFINITY;
    const int jmax = (min(qb * BQ + BQ, L) - 1) / BK;
    int nkept = 0;
    uint32_t word = 0;
    if (bits && tid == 0)
        for (int w = (jmax >> 5) + 1; w < words; ++w) bits[(bh * nqb + qb) * long(words) + w] = 0u;
    for (int t = jmax; t >= 0; --t) {
        const int c0 = t * BK;
        __syncthreads();
        for (int e = tid; e < BK * D; e += BQ) {
            const int jj = e / D, c = e % D;
            const bool ok = c0 + jj < L;
            ks[jj][c] = ok ? k[base + long(c0 + jj) * D + c] : 0.f;
            vs[jj][c] = ok ? v[base + long(c0 + jj) * D + c] : 0.f;
        }
        __syncthreads();
        bool keep = true;
        if (GATED) {
            bool vote = false;
            for (int jj = 0; jj < BK; ++jj) {
                if (!valid || c0 + jj > row) continue;
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < D; ++c) dot = fmaf(qr[c], ks[jj][c], dot);
                vote |= dot >= th;
            }
            keep = __syncthreads_or(vote) != 0;
        }
        if (tid == 0) {
            nkept += keep;
            if (keep) word |= 1u << (t & 31);
            if (bits && ((t & 31) == 0 || t == 0)) {
                bits[(bh * nqb + qb) * long(words) + (t >> 5)] = word;
                word = 0;
            }
        }
        if (!keep) continue;
        for (int jj = 0; jj < BK; ++jj) {
            if (!valid || c0 + jj > row) continue;
            float dot = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                dot = fmaf(qr[c], ks[jj][c], dot);
                dp = fmaf(dr[c], vs[jj][c], dp);
            }
            const float p = fast_exp2(dot * scale_log2 - l2);
            const float dsv = p * (dp - Di) * scale;
#pragma unroll
            for (int c = 0; c < D; ++c) g[c] = fmaf(dsv, ks[jj][c], g[c]);
        }
    }
    if (valid) {
#pragma unroll
        for (int c = 0; c < D; ++c) dq[base + long(row) * D + c] = g[c];
    }
    if (tid == 0) {
        if (kept) kept[bh * nqb + qb] = nkept;
        if (legal) legal[bh * nqb + qb] = jmax + 1;
    }
}

// ----------------------------------------------------------------- launchers
hipError_t launch_simple_fwd_f32(const FwdArgs& a, hipStream_t s) {
    constexpr int BQ = 64, BK = 64, D = 64;
    dim3 grid(a.nqb, a.B * a.H), block(BQ);
    if (a.gated)
        hipLaunchKernelGGL((simple_fwd_f32<BQ, BK, D, true>), grid, block, 0, s, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.L, a.nqb, a.scale_log2,
                           a.log2_tau, a.kept, a.legal, a.bits, a.words);
    else
        hipLaunchKernelGGL((simple_fwd_f32<BQ, BK, D, false>), grid, block, 0, s, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.L, a.nqb, a.scale_log2,
                           a.log2_tau, a.kept, a.legal, a.bits, a.words);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t s) {
    const long rows = long(a.B) * a.H * a.L;
    if (a.f32) {
        const int per_block = 4;  // one wave per row
        dim3 grid(unsigned((rows + per_block - 1) / per_block)), block(64 * per_block);
        hipLaunchKernelGGL((bwd_prep<float, 64>), grid, block, 0, s, (const float*)a.o, (const float*)a.dout,
                           a.lse, a.Dv, a.lse2, a.thr, rows, a.L, a.scale_log2, a.log2_tau);
    } else {
        dim3 grid(unsigned((rows + 15) / 16)), block(256);  // 16 rows per workgroup
        hipLaunchKernelGGL(bwd_prep_bf16_d128, grid, block, 0, s, (const bf16_t*)a.o, (const bf16_t*)a.dout, a.lse,
                           a.Dv, a.lse2, a.thr, rows, a.L, a.scale_log2, a.log2_tau);
    }
    return hipGetLastError();
}

hipError_t launch_simple_bwd_f32(const BwdArgs& a, hipStream_t s) {
    constexpr int BQ = 64, BK = 64, D = 64;
    dim3 g1(a.ntiles, a.B * a.H), b1(BK);
    dim3 g2(a.nqb, a.B * a.H), b2(BQ);
    hipError_t e = mark(a.ev[1], s);
    if (e != hipSuccess) return e;
    if (a.gated) {
        hipLaunchKernelGGL((simple_bwd_dkdv_f32<BQ, BK, D, true>), g1, b1, 0, s, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.Dv, a.lse2, a.thr,
                           (float*)a.dk, (float*)a.dv, a.L, a.nqb, a.ntiles, a.scale, a.scale_log2, a.aux_bits,
                           a.words);
        e = mark(a.ev[2], s);
        hipLaunchKernelGGL((simple_bwd_dq_f32<BQ, BK, D, true>), g2, b2, 0, s, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.Dv, a.lse2, a.thr,
                           (float*)a.dq, a.L, a.nqb, a.scale, a.scale_log2, a.kept, a.legal, a.bits, a.words);
    } else {
        hipLaunchKernelGGL((simple_bwd_dkdv_f32<BQ, BK, D, false>), g1, b1, 0, s, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.Dv, a.lse2, a.thr,
                           (float*)a.dk, (float*)a.dv, a.L, a.nqb, a.ntiles, a.scale, a.scale_log2, a.aux_bits,
                           a.words);
        e = mark(a.ev[2], s);
        hipLaunchKernelGGL((simple_bwd_dq_f32<BQ, BK, D, false>), g2, b2, 0, s, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.Dv, a.lse2, a.thr,
                           (float*)a.dq, a.L, a.nqb, a.scale, a.scale_log2, a.kept, a.legal, a.bits, a.words);
    }
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = mark(a.ev[3], s);
    return e;
}

// Zero n 32-bit words (a fill kernel rather than hipMemsetAsync, so that the
// clear is an ordinary kernel node if the caller captures the call in a graph).
__global__ __launch_bounds__(256) void zero_u32(uint32_t* __restrict__ p, long n) {
    for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n; i += long(gridDim.x) * 256) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, long n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const long blocks = min((n + 255) / 256, 4096L);
    hipLaunchKernelGGL(zero_u32, dim3(unsigned(blocks)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace mala
