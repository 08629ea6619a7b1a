// MALA split-KV decode, bf16 KV cache, head dim 128, 64-key tiles.
//
// Source: "MassAlloc Attention: Let Attention Allocate Its Own Compute"
// (agihunt.info digest).  Threshold paragraph: the same tau and the same
// per-tile test serve decoding; Lq of the new token is the number of cached
// keys it sees (Lk).  Forward paragraph: tiles are visited from the most
// recent keys back with a running normalizer and the first visited tile is
// kept.  Savings and limitations paragraphs: the KV cache is read in full for
// QK; a skipped tile saves its V read, so decode is bound by cache traffic.
//
// One workgroup (4 waves) per (sequence, KV head, partition).  The G query
// heads sharing the KV head are the rows of the workgroup; they share every
// K/V tile load.  Votes run over groups of rpv consecutive rows (rpv = G: the
// whole group, so a skipped tile really saves the V bytes; rpv = 1: one vote
// per query head).  A tile is kept for a vote group iff one of its rows votes
// keep; only that group's rows update their state, and V is read iff some
// group keeps the tile.  The kernel is
// HBM-bound: K tiles are prefetched one tile ahead into registers; V is read
// only for kept tiles.
//
// Thread mapping.  Scores: thread t handles key t/4 of the tile and a
// 32-element quarter of d (four 16-byte loads), bf16 dot2 products in fp32,
// summed over the 4 quarters with lane shuffles; the query quarters are read
// from LDS (every thread of a quarter reads the same addresses).  PV: thread t handles an
// 8-element d chunk (t%16) of keys 16*wave + 4*i + (t/16)%4, i = 0..3; its
// fp32 accumulators are summed over the 16 key subsets once per partition.
// Partial states (m2 = running max of s*log2(e), l, acc[d]) are written per
// (sequence, query head, partition) and merged exactly by the combine kernel.
//
// Partitions.  Plain: partition p holds keys [p*S, min((p+1)*S, Lk)).
// Seeded: tiles stay the 64-key tiles counted from key 0, but partition p
// holds the S/64 tiles ending S/64*p tiles before the newest tile (partition
// 0 is the newest; the oldest may be short).  A seeded decode runs in two
// launches: partition 0 from an empty state, then every older partition with
// partition 0's final (m2, l) added to its test normalizer (the normalizer
// established on the most recent keys, extended across partitions).  Its own
// output state still starts empty, so the exact merge counts no key twice,
// and no tile is kept by force.
#include <float.h>

#include "mala_kernels.hpp"

namespace mala {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// SEED: this launch covers the older partitions of a seeded decode and reads
// partition 0's final state from `part` (written by the previous launch).
// PREV: V tiles are fetched one tile ahead together with K, whatever the
// vote decides.  Used for the newest partition alone (one workgroup per
// sequence and KV head, keeping nearly every tile): there the V load would
// otherwise add a memory latency per tile to a short, serial launch.
// Occupancy: four workgroups per CU (at most 128 VGPRs, so the query rows
// live in LDS) give the HBM stream enough independent tiles in flight; the
// PREV launch runs one workgroup per (sequence, KV head) and keeps the
// registers its extra V prefetch needs instead.
template <int G, bool GATED, bool STATS, bool SEED, bool PREV>
__global__ __launch_bounds__(256, PREV ? 1 : 4) void decode_split_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    float* __restrict__ part, int Hq, int Hkv, int Lk, int Lcap, int split_keys, int nsplit, int tps, int words,
    float scale_log2, float log2_tau, float log2_lq, int32_t* __restrict__ kept, int32_t* __restrict__ legal,
    uint32_t* __restrict__ bits, int pbase, int seeded_grid, int rpv, float* __restrict__ tstat) {
    constexpr int D = 128, BK = 64;
    __shared__ int vote_sm[2][4];
    __shared__ float wmax_sm[2][4][G];
    __shared__ float wsum_sm[2][4][G];
    __shared__ float p_sm[2][G][BK];
    __shared__ float red_sm[G][16][D + 4];
    __shared__ __attribute__((aligned(16))) uint32_t q_sm[G][D / 2];  // the G query rows (bf16 pairs)

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int p = int(blockIdx.x) + pbase;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int b = bg / Hkv, g = bg % Hkv;
    const long kvbase = long(bg) * Lcap * D;
    int k0, k1;
    if (seeded_grid) {
        const int jd = (Lk - 1) / BK;  // tile of the newest key
        const int hi = jd - p * tps;
        const int lo = max(0, hi - tps + 1);
        k0 = lo * BK;
        k1 = min(hi * BK + BK, Lk);
    } else {
        k0 = p * split_keys;
        k1 = min(k0 + split_keys, Lk);
    }
    const int nt = (k1 - k0 + BK - 1) / BK;
    // vote groups: row r belongs to group r / rpv; gm[r] = bits of its group's rows
    const int nvg = G / rpv;
    uint32_t gm[G];
#pragma unroll
    for (int r = 0; r < G; ++r) gm[r] = ((1u << rpv) - 1u) << (r / rpv * rpv);

    // score mapping
    const int skey = tid >> 2, quarter = tid & 3;
    if (tid < G * 16) {  // 16-byte pieces of the G rows
        const int r = tid >> 4, c = tid & 15;
        *reinterpret_cast<u32x4*>(&q_sm[r][4 * c]) =
            *reinterpret_cast<const u32x4*>(q + (long(b) * Hq + g * G + r) * D + 8 * c);
    }
    __syncthreads();
    // PV mapping
    const int dch = tid & 15, ksub = (tid >> 4) & 3;
    float acc[G][8];
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
    // (m2, lsum): this partition's own state; ltest: the normalizer the test
    // uses, which also holds the seed (the same as lsum without one)
    float m2[G], lsum[G], ltest[G];
#pragma unroll
    for (int r = 0; r < G; ++r) { m2[r] = -INFINITY; lsum[r] = 0.f; ltest[r] = 0.f; }
    if (SEED) {
#pragma unroll
        for (int r = 0; r < G; ++r) {
            const float* sp = part + (long(b) * Hq + g * G + r) * nsplit * (D + 2);  // partition 0
            m2[r] = sp[0];
            ltest[r] = sp[1];
        }
    }

    const u32x4 z4 = {0u, 0u, 0u, 0u};
    u32x4 kr[4];
    auto load_k = [&](int t) {
        const int key = k0 + t * BK + skey;
        const bf16_t* src = kc + kvbase + long(key) * D + 32 * quarter;
#pragma unroll
        for (int c = 0; c < 4; ++c) kr[c] = key < k1 ? *reinterpret_cast<const u32x4*>(src + 8 * c) : z4;
    };

    // statistics of vote group tid (threads 0 .. nvg-1), at unit (bg*nvg + tid, p)
    const long sidx = (long(bg) * nvg + tid) * nsplit + p;
    int nkept = 0;
    uint32_t word = 0;
    if (STATS && bits && tid < nvg)
        for (int w = ((nt - 1) >> 5) + 1; w < words; ++w) bits[sidx * words + w] = 0u;

    u32x4 vn[4] = {z4, z4, z4, z4};  // PREV: V of the next tile to visit
    auto load_v = [&](int t, u32x4* dst) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int vk = k0 + t * BK + 16 * wave + 4 * i + ksub;
            dst[i] = vk < k1 ? *reinterpret_cast<const u32x4*>(vc + kvbase + long(vk) * D + 8 * dch) : z4;
        }
    };
    load_k(nt - 1);
    if (PREV) load_v(nt - 1, vn);
    for (int t = nt - 1; t >= 0; --t) {
        const int par = t & 1;
        u32x4 kcur[4] = {kr[0], kr[1], kr[2], kr[3]};
        u32x4 vcur[4] = {vn[0], vn[1], vn[2], vn[3]};
        if (t > 0) {
            load_k(t - 1);
            if (PREV) load_v(t - 1, vn);
        }
        const int key = k0 + t * BK + skey;
        const bool kvalid = key < k1;
        float s[G];
#pragma unroll
        for (int r = 0; r < G; ++r) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 qx = *reinterpret_cast<const u32x4*>(&q_sm[r][16 * quarter + 4 * c]);
                a = dot2(qx[0], kcur[c][0], a);
                a = dot2(qx[1], kcur[c][1], a);
                a = dot2(qx[2], kcur[c][2], a);
                a = dot2(qx[3], kcur[c][3], a);
            }
            a += __shfl_xor(a, 1, 64);
            a += __shfl_xor(a, 2, 64);
            s[r] = kvalid ? a : -INFINITY;
        }

        // per-row maximum over the wave's keys (wave-uniform): the vote tests it,
        // and a kept tile's statistics need it; both go out in one exchange
        float mx[G];
#pragma unroll
        for (int r = 0; r < G; ++r) {
            float x = s[r];
#pragma unroll
            for (int m = 4; m <= 32; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
            mx[r] = x;
        }
        uint32_t rk = (1u << G) - 1u;  // rows whose vote group keeps the tile
        if (GATED) {
            uint32_t vm = 0;  // rows of this wave's keys that vote keep
#pragma unroll
            for (int r = 0; r < G; ++r) {
                const float lz = SEED ? ltest[r] : lsum[r];
                const float thr = (lz == 0.f) ? -FLT_MAX : (m2[r] + fast_log2(lz) + log2_tau - log2_lq) / scale_log2;
                if (mx[r] >= thr) vm |= 1u << r;
            }
            if (lane == 0) {
                vote_sm[par][wave] = int(vm);
#pragma unroll
                for (int r = 0; r < G; ++r) wmax_sm[par][wave][r] = mx[r];
            }
            __syncthreads();
            const uint32_t rv = uint32_t(vote_sm[par][0] | vote_sm[par][1] | vote_sm[par][2] | vote_sm[par][3]);
            rk = 0;
#pragma unroll
            for (int r = 0; r < G; ++r)
                if (rv & gm[r]) rk |= 1u << r;
            if (STATS && tstat && tid < nvg) {
                // log2 of the vote group's test statistic: the largest margin
                // c*max_j s_rj - (m2 + log2 l + log2 tau - log2 Lq) of its rows,
                // from the state the vote used (+inf for an empty state)
                float dl = -INFINITY;
#pragma unroll
                for (int r = 0; r < G; ++r) {
                    if (r / rpv != tid) continue;
                    const float tm = fmaxf(fmaxf(wmax_sm[par][0][r], wmax_sm[par][1][r]),
                                           fmaxf(wmax_sm[par][2][r], wmax_sm[par][3][r]));
                    const float lz = SEED ? ltest[r] : lsum[r];
                    float dr;
                    if (tm == -INFINITY) dr = -INFINITY;
                    else if (lz == 0.f) dr = INFINITY;
                    else dr = tm * scale_log2 - (m2[r] + fast_log2(lz) + log2_tau - log2_lq);
                    dl = fmaxf(dl, dr);
                }
                tstat[sidx * tps + t] = dl;
            }
        } else if (STATS && tstat && tid < nvg) {
            tstat[sidx * tps + t] = NAN;  // tau = 0 runs no test
        }
        if (STATS && tid < nvg) {
            const bool gk = (rk >> (tid * rpv)) & 1u;
            nkept += gk;
            if (gk) word |= 1u << (t & 31);
            if (bits && (t & 31) == 0) {
                bits[sidx * words + (t >> 5)] = word;
                word = 0;
            }
        }
        if (rk == 0) continue;

        // V loads for this tile (consumed after the normalizer update)
        u32x4 vr[4];
        if (PREV) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vr[i] = vcur[i];
        } else {
            load_v(t, vr);
        }
        if (!GATED) {  // (gated: the maxima went out with the vote)
            if (lane == 0)
#pragma unroll
                for (int r = 0; r < G; ++r) wmax_sm[par][wave][r] = mx[r];
            __syncthreads();
        }
        float alpha[G];
#pragma unroll
        for (int r = 0; r < G; ++r) {
            // a row whose group skips the tile keeps its state: alpha = 1, no probability
            const bool rkeep = (rk >> r) & 1u;
            const float tm = fmaxf(fmaxf(wmax_sm[par][0][r], wmax_sm[par][1][r]),
                                   fmaxf(wmax_sm[par][2][r], wmax_sm[par][3][r]));
            const float mn = rkeep ? fmaxf(m2[r], tm * scale_log2) : m2[r];  // kept: finite (a valid key)
            alpha[r] = rkeep ? fast_exp2(m2[r] - mn) : 1.f;
            m2[r] = mn;
            const float pv = rkeep ? fast_exp2(fmaf(s[r], scale_log2, -mn)) : 0.f;  // invalid key (-inf): 0
            float ps = (quarter == 0) ? pv : 0.f;
#pragma unroll
            for (int m = 4; m <= 32; m <<= 1) ps += __shfl_xor(ps, m, 64);
            if (quarter == 0) p_sm[par][r][skey] = pv;
            if (lane == 0) wsum_sm[par][wave][r] = ps;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < G; ++r) {
            const float tsum = (wsum_sm[par][0][r] + wsum_sm[par][1][r]) + (wsum_sm[par][2][r] + wsum_sm[par][3][r]);
            lsum[r] = lsum[r] * alpha[r] + tsum;
            if (SEED) ltest[r] = ltest[r] * alpha[r] + tsum;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] *= alpha[r];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = 16 * wave + 4 * i + ksub;
            float vf[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                vf[2 * c] = __uint_as_float(vr[i][c] << 16);
                vf[2 * c + 1] = __uint_as_float(vr[i][c] & 0xffff0000u);
            }
#pragma unroll
            for (int r = 0; r < G; ++r) {
                const float pw = p_sm[par][r][kk];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(pw, vf[c], acc[r][c]);
            }
        }
        // (no barrier here: the next tile writes the other parity's buffers, and
        // this parity's again only after the next tile's own barrier, which
        // every thread reaches after its reads here)
    }

    // sum the 16 key subsets of every d chunk, write the partial state
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) red_sm[r][4 * wave + ksub][8 * dch + c] = acc[r][c];
    __syncthreads();
    for (int e = tid; e < G * D; e += 256) {
        const int r = e / D, dd = e % D;
        float x = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) x += red_sm[r][u][dd];
        float* dst = part + ((long(b) * Hq + g * G + r) * nsplit + p) * (D + 2);
        dst[2 + dd] = x;
        if (dd == 0) { dst[0] = m2[r]; dst[1] = lsum[r]; }
    }
    if (STATS && tid < nvg) {
        if (kept) kept[sidx] = nkept;
        if (legal) legal[sidx] = nt;
    }
}

// Exact merge of the partition states of every (sequence, query head).
__global__ __launch_bounds__(128) void decode_combine_d128(const float* __restrict__ part, bf16_t* __restrict__ o,
                                                           float* __restrict__ lse, int nsplit) {
    constexpr int D = 128;
    const long bh = blockIdx.x;
    const int dd = threadIdx.x;
    const float* src = part + bh * nsplit * (D + 2);
    float M = -INFINITY;
    for (int p = 0; p < nsplit; ++p) M = fmaxf(M, src[p * (D + 2)]);
    float lam = 0.f, x = 0.f;
    for (int p = 0; p < nsplit; ++p) {
        const float w = fast_exp2(src[p * (D + 2)] - M);
        lam = fmaf(src[p * (D + 2) + 1], w, lam);
        x = fmaf(src[p * (D + 2) + 2 + dd], w, x);
    }
    o[bh * D + dd] = f32_to_bf16(x / lam);
    if (lse && dd == 0) lse[bh] = (M + fast_log2(lam)) * kLn2;
}

template <int G, bool GT, bool ST, bool SD, bool PV = false>
static void launch_decode_one(const DecArgs& a, hipStream_t s, int nparts, int pbase) {
    hipLaunchKernelGGL((decode_split_bf16_d128<G, GT, ST, SD, PV>), dim3(nparts, a.B * a.Hkv), dim3(256), 0, s,
                       (const bf16_t*)a.q, (const bf16_t*)a.kc, (const bf16_t*)a.vc, a.part, a.Hq, a.Hkv, a.Lk,
                       a.Lcap, a.split_keys, a.nsplit, a.tps, a.words, a.scale_log2, a.log2_tau, a.log2_lq, a.kept,
                       a.legal, a.bits, pbase, a.seeded ? 1 : 0, a.rpv, a.tstat);
}

template <int G, bool ST>
static void launch_decode_gs(const DecArgs& a, hipStream_t s) {
    if (!a.gated) {
        launch_decode_one<G, false, ST, false>(a, s, a.nsplit, 0);
    } else if (!a.seeded) {
        launch_decode_one<G, true, ST, false>(a, s, a.nsplit, 0);
    } else {
        // partition 0 first; the older partitions read its final state
        launch_decode_one<G, true, ST, false, true>(a, s, 1, 0);
        if (a.nsplit > 1) launch_decode_one<G, true, ST, true>(a, s, a.nsplit - 1, 1);
    }
}

template <int G>
static void launch_decode_g(const DecArgs& a, hipStream_t s) {
    if (a.kept || a.legal || a.bits || a.tstat) launch_decode_gs<G, true>(a, s);
    else launch_decode_gs<G, false>(a, s);
}

hipError_t launch_decode_bf16(const DecArgs& a, hipStream_t s) {
    switch (a.G) {
        case 1: launch_decode_g<1>(a, s); break;
        case 2: launch_decode_g<2>(a, s); break;
        case 4: launch_decode_g<4>(a, s); break;
        case 8: launch_decode_g<8>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_d128, dim3(a.B * a.Hq), dim3(128), 0, s, a.part, (bf16_t*)a.o, a.lse,
                       a.nsplit);
    return hipGetLastError();
}

}  // namespace mala
