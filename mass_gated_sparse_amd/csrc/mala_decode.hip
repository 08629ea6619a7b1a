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
// One wave per (sequence, KV head, partition).  The G query heads sharing
// the KV head are the rows of the wave's products; they share every K/V tile
// load.  Votes run over groups of rpv consecutive rows (rpv = G: the whole
// group, so a skipped tile really saves the V bytes; rpv = 1: one vote per
// query head).  A tile is kept for a vote group iff one of its rows votes
// keep; only that group's rows update their state, and V is read iff some
// group keeps the tile.  The kernel is HBM-bound: K is requested two tiles
// ahead; V is read only for kept tiles.  Scores and PV are bf16 MFMAs with fp32 accumulation (the
// probabilities enter PV rounded to bf16, the normalizer sums them in fp32);
// the lane mapping is described at the kernel.
// Partial states (m2 = running max of s*log2(e), l, acc[d]) are written per
// (sequence, query head, partition) and merged exactly by the combine kernel.
//
// Partitions.  Plain: partition p holds keys [p*S, min((p+1)*S, Lk)).
// Seeded: tiles stay the 64-key tiles counted from key 0, but partition p
// holds the S/64 tiles ending S/64*p tiles before the newest tile (partition
// 0 is the newest; the oldest may be short).  A seeded decode runs
// partition 0 from an empty state first, then every older partition with
// partition 0's final (m2, l) added to its test normalizer (the normalizer
// established on the most recent keys, extended across partitions).  Its own
// output state still starts empty, so the exact merge counts no key twice,
// and no tile is kept by force.
//
// Partition 0 of a seeded decode with older partitions is not walked tile by
// tile: its tiles' states (m_t, l_t, acc_t) are formed in parallel, each from
// an empty state (the split kernel, ungated, one tile per partition), and
// decode_seed_scan_d128 then visits them newest first, tests each against
// the running state (m2 + log2 l + log2 tau - log2 Lq against the tile's
// c*max s, the split kernel's test) and merges the kept ones.  The same
// decisions and the same state, up to the rounding of the merge order.
#include <float.h>

#include <type_traits>

#include "mala_kernels.hpp"

namespace mala {

// Cross-lane steps that stay off the LDS pipe: a lane's value combined with
// those of the lanes at the same position in the other three 16-lane rows,
// as op(op(row 0, row 1), op(row 2, row 3)).  The row swaps
// (v_permlane16_swap / v_permlane32_swap with both operands x) leave the two
// rows of each pair in the two results; the operations commute, so all four
// lanes hold the same bits.
__device__ __forceinline__ void row_pairs(float x, float& a, float& b, bool wide) {
    const auto s = wide ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                        : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(s[0]);
    b = __uint_as_float(s[1]);
}
__device__ __forceinline__ float rows_max(float x) {
    float a, b;
    row_pairs(x, a, b, false);
    row_pairs(fmaxf(a, b), a, b, true);
    return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum(float x) {
    float a, b;
    row_pairs(x, a, b, false);
    row_pairs(a + b, a, b, true);
    return a + b;
}

// One wave per (partition, sequence, KV head) runs every step of a tile.
// The scores and the PV product are 16x16x32 bf16 MFMAs in which lane
// column n = lane % 16 is query row n (rows past G are zero and never
// written), so a row's state (m2, l, its test threshold) lives in the four
// lanes n, n+16, n+32, n+48 and needs no exchange between waves:
//  - scores S^T (16 keys x 16 rows per chunk, four chunks a tile): A = the
//    chunk's K (lane (key n, g4 = lane/16) holds d 32c+8g4 .. +8 of its key
//    for product c), B = Q^T (lane (row n, g4) the same d of its row); lane
//    (row n, g4) gets keys 16*chunk + 4*g4 + i, i = 0..3;
//  - the tile's row maximum is a max over a lane's 16 scores and the four
//    lanes of the row (row swaps); the vote is one ballot;
//  - PV as O^T (d x rows) += V^T P^T over two 32-key products: B = P^T
//    (lane (row n, g4) holds keys 32h + 16(j/4) + 4*g4 + j%4, j = 0..7: the
//    lane's own probabilities of chunks 2h and 2h+1, rounded to bf16), A =
//    V^T, read from the wave's V tile in LDS by transposing reads (lane
//    (m, g4) gets d = 16*db + m of those eight keys for product db); lane
//    (row n, g4) then holds O[n][16*db + 4*g4 + r] in register r of
//    accumulator db, so the rescale by the row's alpha is lane-local too.
// Memory: K tiles go to registers two tiles ahead (a two-slot ring, tile t
// in slot (nt-1-t) % 2); a kept tile's V goes straight to LDS (direct loads,
// the 16-byte chunks of each 256-byte key row swizzled) right after the vote,
// then the slot the scores have read is refilled with tile t-2, so the wait
// for V before the PV products leaves those 16 K loads in flight.  Every
// tile of the loop issues its 16 refill loads (past tile 0 they read a few
// bytes of the query rows instead, unused): with no load under a branch the
// compiler's own waits for K stay exact.  The V wait counts on those 16
// loads being issued after the V loads and executed; the final tile of an
// odd count refills nothing and waits for every load.  At two waves per
// SIMD a wave keeps 32-48 KiB of K and V in flight, also through runs of
// skipped tiles; the arithmetic of a tile is a few hundred cycles.
// SEED: this launch covers the older partitions of a seeded decode and reads
// partition 0's final state from `part` (written by the previous launch).
// VPF: V of the next tile is requested once the current PV has read the LDS
// tile, whatever the vote decides (the tile states of a seeded decode's
// newest partition, one tile each, and its walk when that runs tile by tile).
template <bool GATED, bool STATS, bool SEED, bool VPF>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kcache, const bf16_t* __restrict__ vcache,
    float* __restrict__ part, int Hq, int Hkv, int G, int Lk, int Lcap, int split_keys, int nsplit, int tps, int words,
    float scale_log2, float log2_tau, float log2_lq, int32_t* __restrict__ kept, int32_t* __restrict__ legal,
    uint32_t* __restrict__ bits, int pbase, int seeded_grid, int rpv, float* __restrict__ tstat) {
    constexpr int D = 128, BK = 64;
    __shared__ __attribute__((aligned(1024))) uint8_t vsm[BK * D * 2];  // V tile: 64 swizzled rows
    const int lane = threadIdx.x, n = lane & 15, g4 = lane >> 4;
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
    const bool live = n < G;  // lane column n is query row n
    const long qrow = long(b) * Hq + g * G + (live ? n : 0);

    u32x4 qf[4];  // Q^T operands; rows past G are zero
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        qf[c] = u32x4{0u, 0u, 0u, 0u};
        if (live) qf[c] = *reinterpret_cast<const u32x4*>(q + qrow * D + 32 * c + 8 * g4);
    }

    // Loads are clamped: a key past the partition (k1 > k0 always) reads the
    // partition's last key instead; its score is set to -inf, so its
    // probability is 0.
    u32x4 kf[2][4][4];  // [slot][chunk][product]
    // (t < 0: no such tile; the loads read the first 128 elements of q)
    auto load_k = [&](auto slot_tag, int t) {
        constexpr int SL = decltype(slot_tag)::value;
        const int tb = k0 + t * BK;
        const bf16_t* base = t >= 0 ? kcache + kvbase + long(tb) * D : q;
        const int lim = t >= 0 ? k1 - 1 - tb : 0;  // last key of the partition, tile-relative
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const bf16_t* src = base + min(16 * ch + n, lim) * D + 8 * g4;
#pragma unroll
            for (int c = 0; c < 4; ++c) kf[SL][ch][c] = *reinterpret_cast<const u32x4*>(src + 32 * c);
        }
    };
    // V tile t into LDS: load i writes keys 4i .. 4i+3, lane l the chunk at
    // swizzled position l % 16 of key 4i + l/16
    const uint32_t vlds = lds_addr_of(vsm);
    auto load_v = [&](int t) {
        const int tb = k0 + t * BK;
        const int lim = k1 - 1 - tb;  // last key of the partition, tile-relative
        const bf16_t* base = vcache + kvbase + long(tb) * D;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kl = 4 * i + g4;
            const uint32_t ch = uint32_t(n ^ rowkey(kl));
            dma16s(base, uint32_t(min(kl, lim)) * 256u + ch * 16u, vlds + 1024u * i);
        }
    };
    // transposing-read offsets: lane (m = n, g4) addresses key 4*g4 + m/4
    // (+ 32h + 16 for the second half of product h) at d = 16*db + 4*(m%4)
    int vrd[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) vrd[db] = swz_el(4 * g4 + (n >> 2), 16 * db + 4 * (n & 3));

    // (m2, lsum): this partition's own state of row n; ltest: the normalizer
    // the test uses, which also holds the seed (the same as lsum without one)
    float m2 = -INFINITY, lsum = 0.f, ltest = 0.f;
    if (SEED && live) {
        const float* sp = part + qrow * nsplit * (D + 2);  // partition 0
        m2 = sp[0];
        ltest = sp[1];
    }
    // The row's test threshold in the raw dot-product domain,
    // (m2 + log2 l + log2 tau - log2 Lq) / c with l the test normalizer,
    // recomputed only after a tile its vote group keeps; an empty state keeps
    // any visible key.
    const float inv_scale_log2 = 1.f / scale_log2;
    auto thr_of = [&]() {
        const float lz = SEED ? ltest : lsum;
        return (lz == 0.f) ? -FLT_MAX : (m2 + fast_log2(lz) + log2_tau - log2_lq) * inv_scale_log2;
    };

    // statistics of vote group n / rpv: kept by lane n = its first row (g4 = 0)
    const int nvg = G / rpv;
    const bool lead = g4 == 0 && live && n % rpv == 0;
    const long sidx = (long(bg) * nvg + n / rpv) * nsplit + p;
    int nkept = 0;
    uint32_t word = 0;
    if (STATS && bits && lead)
        for (int w = ((nt - 1) >> 5) + 1; w < words; ++w) bits[sidx * words + w] = 0u;

    f32x4 acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    load_k(S0{}, nt - 1);
    load_k(S1{}, nt - 2);
    if (VPF) load_v(nt - 1);
    float thr = thr_of();  // (after the first requests: a seed load's latency overlaps them)
    // LAST: the final tile after the pairs of the loop; it refills nothing
    // (the refill would be dead code, which the compiler drops)
    auto tile = [&](auto slot_tag, auto last_tag, int t) {
        constexpr int SL = decltype(slot_tag)::value;
        constexpr bool LAST = decltype(last_tag)::value;
        f32x4 s[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            s[ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) s[ch] = mfma16(kf[SL][ch][c], qf[c], s[ch]);
        }
        if (k0 + t * BK + BK > k1) {  // the partition's newest tile may be partial
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + t * BK + 16 * ch + 4 * g4 + i >= k1) s[ch][i] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
        for (int ch = 1; ch < 4; ++ch) mx = fmaxf(mx, fmaxf(fmaxf(s[ch][0], s[ch][1]), fmaxf(s[ch][2], s[ch][3])));
        mx = rows_max(mx);  // the row's maximum over the tile (raw dot product)

        uint32_t rk = (1u << G) - 1u;  // rows whose vote group keeps the tile
        if (GATED) {
            const uint32_t vm = uint32_t(__ballot(live && mx >= thr)) & 0xffffu;
            rk = 0;
            for (int r0 = 0; r0 < G; r0 += rpv) {
                const uint32_t gmk = ((1u << rpv) - 1u) << r0;
                if (vm & gmk) rk |= gmk;
            }
            if (STATS && tstat) {
                // log2 of the vote group's test statistic: the largest margin
                // c*max_j s_rj - (m2 + log2 l + log2 tau - log2 Lq) of its rows,
                // from the state the vote used (+inf for an empty state)
                const float lz = SEED ? ltest : lsum;
                float dr = (!live || mx == -INFINITY) ? -INFINITY
                           : (lz == 0.f)              ? INFINITY
                                                      : mx * scale_log2 - (m2 + fast_log2(lz) + log2_tau - log2_lq);
                for (int m = 1; m < rpv; m <<= 1) dr = fmaxf(dr, __shfl_xor(dr, m, 64));
                if (lead) tstat[sidx * tps + t] = dr;
            }
        } else if (STATS && tstat && lead) {
            tstat[sidx * tps + t] = NAN;  // tau = 0 runs no test
        }
        if (STATS && lead) {
            const bool gk = (rk >> n) & 1u;
            nkept += gk;
            if (gk) word |= 1u << (t & 31);
            if (bits && (t & 31) == 0) {
                bits[sidx * words + (t >> 5)] = word;
                word = 0;
            }
        }
        if (!VPF && rk != 0) load_v(t);
        if (!LAST) load_k(slot_tag, t - 2);  // into the slot the products have read
        if (rk != 0) {
            // a row whose group skips the tile keeps its state: alpha = 1, no probability
            const bool rkeep = (rk >> n) & 1u;
            const float mn = rkeep ? fmaxf(m2, mx * scale_log2) : m2;  // kept: finite (a valid key)
            const float alpha = rkeep ? fast_exp2(m2 - mn) : 1.f;
            m2 = mn;
            float ps = 0.f;
            u32x4 pb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int ch = 2 * h + (e >> 1), i0 = 2 * (e & 1);
                    const float p0 = rkeep ? fast_exp2(fmaf(s[ch][i0], scale_log2, -mn)) : 0.f;  // -inf: 0
                    const float p1 = rkeep ? fast_exp2(fmaf(s[ch][i0 + 1], scale_log2, -mn)) : 0.f;
                    ps += p0 + p1;
                    pb[h][e] = pack_bf16x2(p0, p1);
                }
            ps = rows_sum(ps);
            lsum = lsum * alpha + ps;
            if (SEED) ltest = ltest * alpha + ps;
            if (GATED && rkeep) thr = thr_of();
            if (alpha != 1.f) {  // (exact: most tiles move no row's maximum)
#pragma unroll
                for (int db = 0; db < 8; ++db)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[db][r] *= alpha;
            }
            // V(t) has landed once at most the K refill's 16 loads (issued after
            // it) are pending
            if (LAST) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const u32x2 lo = tr16(vsm, vrd[db] + 8192 * h);
                    const u32x2 hi = tr16(vsm, vrd[db] + 8192 * h + 4096);
                    acc[db] = mfma16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[h], acc[db]);
                }
        }
        if (VPF && t > 0) load_v(t - 1);  // (the products above have read the LDS tile)
    };
    using MID = std::false_type;
    using LAST = std::true_type;
    int t = nt - 1;
    for (; t >= 1; t -= 2) {
        tile(S0{}, MID{}, t);
        tile(S1{}, MID{}, t - 1);
    }
    if (t == 0) tile(S0{}, LAST{}, 0);
    if (live) {
        float* dst = part + (qrow * nsplit + p) * (D + 2);
        if (g4 == 0) {
            dst[0] = m2;
            dst[1] = lsum;
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            *reinterpret_cast<f32x2*>(dst + 2 + 16 * db + 4 * g4) = f32x2{acc[db][0], acc[db][1]};
            *reinterpret_cast<f32x2*>(dst + 4 + 16 * db + 4 * g4) = f32x2{acc[db][2], acc[db][3]};
        }
    }
    if (STATS && lead) {
        if (kept) kept[sidx] = nkept;
        if (legal) legal[sidx] = nt;
    }
}

// Newest partition of a seeded decode from the states of its tiles (tile
// partition p = tile tps-1-p of the partition, each formed from an empty
// state): one workgroup of 512 threads per (sequence, K/V head).  Lane r < G
// of the first wave replays row r's walk over the tiles, newest first: a vote
// group (rpv consecutive rows) keeps a tile iff one of its rows has
// c*max s >= m2 + log2 l + log2 tau - log2 Lq (any visible key while l = 0),
// and its rows then merge the tile's (m_t, l_t) into their state.  Every
// thread (row mod 4, d) then sums the kept tiles' acc_t with weights
// 2^(m_t - m_final).  Writes partition 0's (m2, l, acc) in the split kernel's
// format, and its statistics.
template <int G, bool STATS>
__global__ __launch_bounds__(512) void decode_seed_scan_d128(
    const float* __restrict__ tpart, float* __restrict__ part, int Hq, int Hkv, int nsplit, int tps, int words,
    float log2_tau, float log2_lq, int rpv, int32_t* __restrict__ kept, int32_t* __restrict__ legal,
    uint32_t* __restrict__ bits, float* __restrict__ tstat) {
    constexpr int D = 128;
    __shared__ float mt_sm[G][kSeedScanMaxTiles], lt_sm[G][kSeedScanMaxTiles];
    __shared__ __attribute__((aligned(16))) float w_sm[G][kSeedScanMaxTiles];  // merge weights (0: skipped)
    __shared__ float fin_sm[2][G];
    const int tid = threadIdx.x, bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
    auto src = [&](int r, int p) { return tpart + ((long(b) * Hq + g * G + r) * tps + p) * (D + 2); };
    for (int e = tid; e < G * tps; e += 512) {
        const int r = e / tps, p = e % tps;
        mt_sm[r][p] = src(r, p)[0];
        lt_sm[r][p] = src(r, p)[1];
    }
    __syncthreads();
    if (tid < 64) {  // the walk: lane r = row r (lanes G.. idle)
        const int r = tid;
        const bool live = r < G;
        const int rc = live ? r : 0;
        const uint64_t gmask = ((rpv >= 64 ? ~0ull : (1ull << rpv) - 1ull)) << (r / rpv * rpv);
        const bool lead = live && r % rpv == 0;  // keeps its group's statistics
        const long sidx = (long(bg) * (G / rpv) + r / rpv) * nsplit;  // partition 0 (lead lanes)
        float m2 = -INFINITY, l = 0.f;
        int nkept = 0;
        uint32_t word = 0;
        for (int p = 0; p < tps; ++p) {
            const int t = tps - 1 - p;
            const float mt = mt_sm[rc][p];
            const float base = m2 + fast_log2(l) + log2_tau - log2_lq;
            const bool v = live && ((l == 0.f) ? (mt != -INFINITY) : (mt >= base));
            const bool keep = (__ballot(v) & gmask) != 0ull;
            if (STATS) {
                float dl = !live || mt == -INFINITY ? -INFINITY : (l == 0.f) ? INFINITY : mt - base;
                for (int m = 1; m < rpv; m <<= 1) dl = fmaxf(dl, __shfl_xor(dl, m, 64));
                if (lead) {
                    nkept += keep;
                    if (keep) word |= 1u << (t & 31);
                    if (bits && (t & 31) == 0) {
                        bits[sidx * words + (t >> 5)] = word;
                        word = 0;
                    }
                    if (tstat) tstat[sidx * tps + t] = dl;
                }
            }
            if (live) {
                if (keep) {
                    const float mn = fmaxf(m2, mt);
                    l = l * fast_exp2(m2 - mn) + lt_sm[rc][p] * fast_exp2(mt - mn);
                    m2 = mn;
                }
                w_sm[r][p] = keep ? 1.f : 0.f;
            }
        }
        if (live) {
            fin_sm[0][r] = m2;
            fin_sm[1][r] = l;
        }
        if (STATS && lead) {
            if (kept) kept[sidx] = nkept;
            if (legal) legal[sidx] = tps;
        }
    }
    __syncthreads();
    for (int e = tid; e < G * tps; e += 512) {
        const int r = e / tps, p = e % tps;
        w_sm[r][p] = w_sm[r][p] != 0.f ? fast_exp2(mt_sm[r][p] - fin_sm[0][r]) : 0.f;
    }
    __syncthreads();
    const int dd = tid & 127;
    for (int r = tid >> 7; r < G; r += 4) {
        float x = 0.f;
        // 32 tiles' loads in flight at a time; a skipped tile weighs 0
        for (int p0 = 0; p0 < tps; p0 += 32) {
            float a32[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) a32[i] = src(r, min(p0 + i, tps - 1))[2 + dd];
#pragma unroll
            for (int i = 0; i < 32; ++i) x = fmaf(a32[i], p0 + i < tps ? w_sm[r][min(p0 + i, tps - 1)] : 0.f, x);
        }
        float* dst = part + ((long(b) * Hq + g * G + r) * nsplit) * (D + 2);
        dst[2 + dd] = x;
        if (dd == 0) {
            dst[0] = fin_sm[0][r];
            dst[1] = fin_sm[1][r];
        }
    }
}

// Exact merge of the partition states of every (sequence, query head).
__global__ __launch_bounds__(128) void decode_combine_d128(const float* __restrict__ part, bf16_t* __restrict__ o,
                                                           float* __restrict__ lse, int nsplit) {
    constexpr int D = 128;
    __shared__ float wmax[2];
    const long bh = blockIdx.x;
    const int dd = threadIdx.x;
    const float* src = part + bh * nsplit * (D + 2);
    // M = max over the partitions, the threads splitting the partitions (their
    // loads are independent, so they are all in flight together)
    float M = -INFINITY;
    for (int p = dd; p < nsplit; p += 128) M = fmaxf(M, src[p * (D + 2)]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    if ((dd & 63) == 0) wmax[dd >> 6] = M;
    __syncthreads();
    M = fmaxf(wmax[0], wmax[1]);
    // weighted sums in partition order; unrolled so several partitions' loads
    // are in flight at once
    float lam = 0.f, x = 0.f;
#pragma unroll 8
    for (int p = 0; p < nsplit; ++p) {
        const float* sp = src + p * (D + 2);
        const float w = fast_exp2(sp[0] - M);
        lam = fmaf(sp[1], w, lam);
        x = fmaf(sp[2 + dd], w, x);
    }
    o[bh * D + dd] = f32_to_bf16(x / lam);
    if (lse && dd == 0) lse[bh] = (M + fast_log2(lam)) * kLn2;
}

template <bool GT, bool ST, bool SD, bool VPF = false>
static void launch_decode_one(const DecArgs& a, hipStream_t s, int nparts, int pbase) {
    hipLaunchKernelGGL((decode_split_bf16_d128<GT, ST, SD, VPF>), dim3(nparts, a.B * a.Hkv), dim3(64), 0, s,
                       (const bf16_t*)a.q, (const bf16_t*)a.kc, (const bf16_t*)a.vc, a.part, a.Hq, a.Hkv, a.G, a.Lk,
                       a.Lcap, a.split_keys, a.nsplit, a.tps, a.words, a.scale_log2, a.log2_tau, a.log2_lq, a.kept,
                       a.legal, a.bits, pbase, a.seeded ? 1 : 0, a.rpv, a.tstat);
}

template <int G, bool ST>
static void launch_decode_gs(const DecArgs& a, hipStream_t s) {
    if (!a.gated) {
        launch_decode_one<false, ST, false>(a, s, a.nsplit, 0);
    } else if (!a.seeded) {
        launch_decode_one<true, ST, false>(a, s, a.nsplit, 0);
    } else if (a.nsplit > 1 && a.tps <= kSeedScanMaxTiles && a.tpart) {
        // partition 0: its tiles' states in parallel (one tile per
        // partition of the tile workspace, ungated), then the replayed walk;
        // then the older partitions, which read its final state
        DecArgs t = a;
        t.part = a.tpart;
        t.nsplit = a.tps;
        t.tps = 1;
        launch_decode_one<false, false, false, true>(t, s, a.tps, 0);
        hipLaunchKernelGGL((decode_seed_scan_d128<G, ST>), dim3(a.B * a.Hkv), dim3(512), 0, s, a.tpart, a.part,
                           a.Hq, a.Hkv, a.nsplit, a.tps, a.words, a.log2_tau, a.log2_lq, a.rpv, a.kept, a.legal,
                           a.bits, a.tstat);
        launch_decode_one<true, ST, true>(a, s, a.nsplit - 1, 1);
    } else {
        // partition 0 walked tile by tile; the older partitions read its final state
        launch_decode_one<true, ST, false, true>(a, s, 1, 0);
        if (a.nsplit > 1) launch_decode_one<true, ST, true>(a, s, a.nsplit - 1, 1);
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
