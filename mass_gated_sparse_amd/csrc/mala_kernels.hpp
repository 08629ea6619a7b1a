// Launch descriptors shared by the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mala_device.hpp"

namespace mala {

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }

struct FwdArgs {
    const void *q, *k, *v;
    void* o;
    float* lse;
    int B, H, Hkv, L, d;  // H query heads, Hkv key/value heads (H % Hkv == 0); L query rows
    int P, Lk, Lkcap;     // first row's key position, valid keys (P + L), K/V rows per head
    int nqb, ntiles, words;
    float scale_log2;  // scale * log2(e)
    float log2_tau;    // log2(tau); +inf for tau = +inf
    bool gated;        // false for tau = 0
    int32_t *kept, *legal;
    uint32_t* bits;
    float* tstat;      // statistics: log2 of each tile's test statistic [B, H, nqb, ceil(Lk/64)]
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float* lse;
    void *dq, *dk, *dv;
    float *Dv, *lse2, *thr;  // per-row workspace arrays [B, H, L]
    uint32_t* dbits;         // workspace: backward decisions [B, H, nqb, words], dQ pass -> dK/dV pass
    int B, H, Hkv, L, d;     // H query heads, Hkv key/value heads (H % Hkv == 0)
    int nqb, ntiles, words;
    float scale, scale_log2, log2_tau;
    bool gated, f32;
    int32_t *kept, *legal;
    uint32_t *bits, *aux_bits;  // aux_bits: the blocks the dK/dV kernel visited (debug)
    float* tstat;               // statistics: log2 of each tile's test statistic [B, H, nqb, ntiles]
    hipEvent_t ev[4];           // optional timing events (see mala_stats)
};

struct DecArgs {
    const void *q, *kc, *vc;
    void* o;
    float* lse;
    float* part;  // [B, Hq, nsplit, d + 2] fp32 partial states (m2, l, acc[d])
    float* tpart;  // seeded: [B, Hq, tps, d + 2] states of partition 0's tiles (or null)
    int B, Hq, Hkv, G, Lk, Lcap, d;
    int split_keys, bk, nsplit, tps, words;
    float scale_log2, log2_tau, log2_lq;
    bool gated;
    bool seeded;  // partitions counted back from the newest tile; older ones seeded with the newest's state
    int rpv;      // query heads per vote (divides G)
    int32_t *kept, *legal;
    uint32_t* bits;
    float* tstat;  // statistics: log2 of each (vote group, tile) test statistic [B, V, nsplit, tps]
};

// Records e on s when e is non-null.
inline hipError_t mark(hipEvent_t e, hipStream_t s) { return e ? hipEventRecord(e, s) : hipSuccess; }

hipError_t launch_simple_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, long n, hipStream_t s);
hipError_t launch_simple_bwd_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecArgs& a, hipStream_t s);
// Largest partition (in tiles) whose seeded newest-partition walk is replayed
// from per-tile states; longer ones are walked tile by tile.
constexpr int kSeedScanMaxTiles = 256;

}  // namespace mala
