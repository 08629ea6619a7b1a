// C ABI of libmala.so: argument validation, workspace layout and dispatch.
// The operator's definition and the contract of every entry point are in
// include/mala.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/mala.h"
#include "mala_kernels.hpp"

// Device scratch of mala_decode_noalloc: the split partial states live here
// instead of in a caller's workspace.  Every GPU the library runs on holds its
// own copy, from the loading of the code object until the process ends.  On
// the host, `scratch` names a host-side stand-in, never device memory: host
// code uses only the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[MALA_DECODE_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

thread_local char g_err[512] = "";

mala_status fail(mala_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

mala_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MALA_OK;
    return fail(MALA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

long cdiv(long a, long b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// tau >= 0 (possibly +inf); NaN and negatives rejected.
bool tau_ok(float tau) { return tau >= 0.f; }

float eff_scale(float scale, int d) { return scale > 0.f ? scale : 1.f / sqrtf(float(d)); }

float log2_tau_of(float tau) { return isinf(tau) ? INFINITY : log2f(tau); }

// Supported prefill instantiations.
bool prefill_supported(mala_dtype dt, int d, mala_tile t) {
    if (dt == MALA_BF16) return d == 128 && t.bq == 128 && t.bk == 64;
    if (dt == MALA_F32) return d == 64 && t.bq == 64 && t.bk == 64;
    return false;
}

mala_status check_prefill(const void* q, const void* k, const void* v, int B, int H, int Hkv, int L, int d,
                          mala_dtype dt, float tau, mala_tile tile) {
    if (!q || !k || !v) return fail(MALA_ERR_INVALID_ARG, "null input pointer");
    if (B <= 0 || H <= 0 || Hkv <= 0 || L <= 0 || d <= 0)
        return fail(MALA_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d Hkv=%d L=%d d=%d)", B, H, Hkv, L, d);
    if (tile.bq <= 0 || tile.bk <= 0) return fail(MALA_ERR_INVALID_ARG, "tile sizes must be positive");
    if (!tau_ok(tau)) return fail(MALA_ERR_INVALID_ARG, "tau must be >= 0 (got %f)", double(tau));
    if (dt != MALA_BF16 && dt != MALA_F32) return fail(MALA_ERR_INVALID_ARG, "unknown dtype %d", int(dt));
    if (H % Hkv) return fail(MALA_ERR_INVALID_ARG, "H (%d) not a multiple of Hkv (%d)", H, Hkv);
    if (H != Hkv && dt != MALA_BF16)
        return fail(MALA_ERR_UNSUPPORTED, "grouped K/V heads (H=%d, Hkv=%d) need bf16", H, Hkv);
    if (!prefill_supported(dt, d, tile))
        return fail(MALA_ERR_UNSUPPORTED, "unsupported prefill instantiation dtype=%d d=%d tile=%dx%d", int(dt), d,
                    tile.bq, tile.bk);
    if ((long)B * H * L * d >= (1L << 40)) return fail(MALA_ERR_UNSUPPORTED, "tensor too large");
    // element offsets within one head are 32-bit in the kernels
    if ((long)L * d >= (1L << 31)) return fail(MALA_ERR_UNSUPPORTED, "sequence too long (L*d >= 2^31)");
    return MALA_OK;
}

}  // namespace

extern "C" {

int mala_version(void) { return 103; }

const char* mala_status_string(mala_status s) {
    switch (s) {
        case MALA_OK: return "ok";
        case MALA_ERR_INVALID_ARG: return "invalid argument";
        case MALA_ERR_UNSUPPORTED: return "unsupported configuration";
        case MALA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* mala_last_error(void) { return g_err; }

mala_status mala_fwd(const void* q, const void* k, const void* v, int B, int H, int Hkv, int L, int d,
                     mala_dtype dtype, float tau, mala_tile tile, float scale, void* o, float* lse,
                     mala_stats* stats, void* stream) {
    g_err[0] = 0;
    mala_status st = check_prefill(q, k, v, B, H, Hkv, L, d, dtype, tau, tile);
    if (st) return st;
    if (!o || !lse) return fail(MALA_ERR_INVALID_ARG, "null output pointer");
    mala::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.Hkv = Hkv; a.L = L; a.d = d;
    a.P = 0; a.Lk = L; a.Lkcap = L;
    a.nqb = int(cdiv(L, tile.bq));
    a.ntiles = int(cdiv(L, tile.bk));
    a.words = int(cdiv(a.ntiles, 32));
    const float sc = eff_scale(scale, d);
    a.scale_log2 = sc * mala::kLog2e;
    a.log2_tau = log2_tau_of(tau);
    a.gated = tau != 0.f;
    if (stats) {
        if (stats->test_stat && dtype != MALA_BF16)
            return fail(MALA_ERR_UNSUPPORTED, "test_stat needs bf16 (not written by the fp32 path)");
        a.kept = stats->kept; a.legal = stats->legal; a.bits = stats->keep_bits; a.tstat = stats->test_stat;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipEvent_t e0 = stats ? (hipEvent_t)stats->events[0] : nullptr, e1 = stats ? (hipEvent_t)stats->events[1] : nullptr;
    hipError_t e = mala::mark(e0, s);
    if (e == hipSuccess) e = dtype == MALA_BF16 ? mala::launch_fwd_bf16(a, s) : mala::launch_simple_fwd_f32(a, s);
    if (e == hipSuccess) e = mala::mark(e1, s);
    return hip_status(e, "mala_fwd launch");
}

mala_status mala_fwd_chunk(const void* q, const void* kcache, const void* vcache, int B, int H, int Hkv, int Lq,
                           int P, int Lcap, int d, mala_dtype dtype, float tau, mala_tile tile, float scale, void* o,
                           float* lse, mala_stats* stats, void* stream) {
    g_err[0] = 0;
    mala_status st = check_prefill(q, kcache, vcache, B, H, Hkv, Lq, d, dtype, tau, tile);
    if (st) return st;
    if (!o || !lse) return fail(MALA_ERR_INVALID_ARG, "null output pointer");
    if (P < 0) return fail(MALA_ERR_INVALID_ARG, "negative chunk offset P=%d", P);
    if ((long)P + Lq > Lcap) return fail(MALA_ERR_INVALID_ARG, "P + Lq (%ld) exceeds Lcap (%d)", (long)P + Lq, Lcap);
    if (dtype != MALA_BF16) return fail(MALA_ERR_UNSUPPORTED, "chunked prefill needs bf16");
    if ((long)B * Hkv * Lcap * d >= (1L << 40)) return fail(MALA_ERR_UNSUPPORTED, "cache too large");
    if ((long)Lcap * d >= (1L << 31)) return fail(MALA_ERR_UNSUPPORTED, "sequence too long (Lcap*d >= 2^31)");
    mala::FwdArgs a{};
    a.q = q; a.k = kcache; a.v = vcache; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.Hkv = Hkv; a.L = Lq; a.d = d;
    a.P = P; a.Lk = P + Lq; a.Lkcap = Lcap;
    a.nqb = int(cdiv(Lq, tile.bq));
    a.ntiles = int(cdiv(a.Lk, tile.bk));
    a.words = int(cdiv(a.ntiles, 32));
    const float sc = eff_scale(scale, d);
    a.scale_log2 = sc * mala::kLog2e;
    a.log2_tau = log2_tau_of(tau);
    a.gated = tau != 0.f;
    if (stats) { a.kept = stats->kept; a.legal = stats->legal; a.bits = stats->keep_bits; a.tstat = stats->test_stat; }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipEvent_t e0 = stats ? (hipEvent_t)stats->events[0] : nullptr, e1 = stats ? (hipEvent_t)stats->events[1] : nullptr;
    hipError_t e = mala::mark(e0, s);
    if (e == hipSuccess) e = mala::launch_fwd_bf16(a, s);
    if (e == hipSuccess) e = mala::mark(e1, s);
    return hip_status(e, "mala_fwd_chunk launch");
}

size_t mala_bwd_workspace_size(int B, int H, int L, int d, mala_dtype dtype, mala_tile tile) {
    (void)d; (void)dtype;
    if (B <= 0 || H <= 0 || L <= 0 || tile.bq <= 0 || tile.bk <= 0) return 0;
    const size_t words = cdiv(cdiv(L, tile.bk), 32);
    return 3 * align256(size_t(B) * H * L * sizeof(float)) +
           align256(size_t(B) * H * cdiv(L, tile.bq) * words * sizeof(uint32_t));
}

mala_status mala_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     int B, int H, int Hkv, int L, int d, mala_dtype dtype, float tau, mala_tile tile, float scale,
                     void* dq, void* dk, void* dv, mala_stats* stats, void* workspace, size_t workspace_bytes,
                     void* stream) {
    g_err[0] = 0;
    mala_status st = check_prefill(q, k, v, B, H, Hkv, L, d, dtype, tau, tile);
    if (st) return st;
    if (!o || !lse || !dout) return fail(MALA_ERR_INVALID_ARG, "null forward-state or dout pointer");
    if (!dq || !dk || !dv) return fail(MALA_ERR_INVALID_ARG, "null gradient pointer");
    const size_t need = mala_bwd_workspace_size(B, H, L, d, dtype, tile);
    if (!workspace || workspace_bytes < need)
        return fail(MALA_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(MALA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    mala::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    const size_t rows = size_t(B) * H * L;
    char* ws = static_cast<char*>(workspace);
    a.Dv = reinterpret_cast<float*>(ws);
    a.lse2 = reinterpret_cast<float*>(ws + align256(rows * 4));
    a.thr = reinterpret_cast<float*>(ws + 2 * align256(rows * 4));
    a.dbits = reinterpret_cast<uint32_t*>(ws + 3 * align256(rows * 4));
    a.B = B; a.H = H; a.Hkv = Hkv; a.L = L; a.d = d;
    a.nqb = int(cdiv(L, tile.bq));
    a.ntiles = int(cdiv(L, tile.bk));
    a.words = int(cdiv(a.ntiles, 32));
    a.scale = eff_scale(scale, d);
    a.scale_log2 = a.scale * mala::kLog2e;
    a.log2_tau = log2_tau_of(tau);
    a.gated = tau != 0.f;
    a.f32 = dtype == MALA_F32;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (stats) {
        if (stats->test_stat && a.f32)
            return fail(MALA_ERR_UNSUPPORTED, "test_stat needs bf16 (not written by the fp32 path)");
        a.kept = stats->kept; a.legal = stats->legal; a.bits = stats->keep_bits; a.tstat = stats->test_stat;
        a.aux_bits = stats->keep_bits_dkdv;
        for (int i = 0; i < 4; ++i) a.ev[i] = (hipEvent_t)stats->events[i];
        if (a.aux_bits) {  // the dK/dV pass ORs in the blocks it visits
            hipError_t e0 = mala::launch_zero_u32(a.aux_bits, long(B) * H * a.nqb * a.words, s);
            if (e0 != hipSuccess) return hip_status(e0, "mala_bwd stats clear");
        }
    }
    hipError_t e = mala::mark(a.ev[0], s);
    if (e == hipSuccess) e = mala::launch_bwd_prep(a, s);
    if (e != hipSuccess) return hip_status(e, "mala_bwd prep launch");
    e = a.f32 ? mala::launch_simple_bwd_f32(a, s) : mala::launch_bwd_bf16(a, s);
    return hip_status(e, "mala_bwd launch");
}

// Partition states of a decode: [B, Hq, nsplit, d + 2] floats.
static size_t decode_part_bytes(int B, int Hq, long nsplit, int d) {
    return align256(size_t(B) * Hq * nsplit * (d + 2) * sizeof(float));
}
// Tile states of a seeded decode's newest partition, when it is replayed from
// them (more than one partition, at most kSeedScanMaxTiles 64-key tiles in
// one): [B, Hq, split_keys / 64, d + 2] floats after the partition states.
static size_t decode_tile_bytes(int B, int Hq, long nsplit, int d, int split_keys) {
    const long tps = split_keys / 64;
    if (nsplit < 2 || split_keys % 64 || tps > mala::kSeedScanMaxTiles) return 0;
    return align256(size_t(B) * Hq * tps * (d + 2) * sizeof(float));
}

size_t mala_decode_workspace_size(int B, int Hq, int Hkv, int Lk, int d, int split_keys) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || d <= 0 || split_keys <= 0) return 0;
    const long nsplit = cdiv(Lk, split_keys);
    return decode_part_bytes(B, Hq, nsplit, d) + decode_tile_bytes(B, Hq, nsplit, d, split_keys);
}

// Address of `scratch` on the current device, looked up once per device
// (with that device current) and kept for the life of the process.
static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static float* g_scratch_dev[kMaxDevices] = {};

static mala_status scratch_of_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "mala_decode_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MALA_ERR_UNSUPPORTED, "mala_decode_noalloc: device ordinal %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "mala_decode_noalloc: hipGetSymbolAddress(scratch)");
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255))
            return fail(MALA_ERR_HIP, "mala_decode_noalloc: scratch address %p unusable", p);
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_dev[dev];
    return MALA_OK;
}

// use_scratch: the partials go to this device's `scratch` (workspace and
// workspace_bytes are ignored), after every argument has been checked.
static mala_status decode_call(const char* name, bool seeded, const void* q, const void* kcache, const void* vcache,
                               int B, int Hq, int Hkv, int Lk, int Lcap, int d, mala_dtype dtype, float tau,
                               int split_keys, int bk, int rows_per_vote, float scale, void* o, float* lse,
                               mala_stats* stats, void* workspace, size_t workspace_bytes, void* stream,
                               bool use_scratch = false) {
    g_err[0] = 0;
    if (!q || !kcache || !vcache || !o) return fail(MALA_ERR_INVALID_ARG, "null pointer");
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || d <= 0 || split_keys <= 0 || bk <= 0)
        return fail(MALA_ERR_INVALID_ARG, "sizes must be positive");
    if (Lcap < Lk) return fail(MALA_ERR_INVALID_ARG, "Lcap (%d) < Lk (%d)", Lcap, Lk);
    if (!tau_ok(tau)) return fail(MALA_ERR_INVALID_ARG, "tau must be >= 0 (got %f)", double(tau));
    if (dtype != MALA_BF16 && dtype != MALA_F32) return fail(MALA_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
    if (Hq % Hkv) return fail(MALA_ERR_INVALID_ARG, "Hq (%d) not a multiple of Hkv (%d)", Hq, Hkv);
    const int G = Hq / Hkv;
    // kernel instantiations exist for G = 1, 2, 4 and 8 query heads per KV head
    const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
    if (dtype != MALA_BF16 || d != 128 || bk != 64 || !g_ok || split_keys % bk)
        return fail(MALA_ERR_UNSUPPORTED, "unsupported decode instantiation dtype=%d d=%d bk=%d G=%d split=%d",
                    int(dtype), d, bk, G, split_keys);
    if (rows_per_vote == 0) rows_per_vote = G;
    if (rows_per_vote < 0 || G % rows_per_vote)
        return fail(MALA_ERR_INVALID_ARG, "rows_per_vote (%d) must divide Hq/Hkv (%d)", rows_per_vote, G);
    // a plain decode needs the partition states only; a seeded one also the
    // tile states of its newest partition
    const long nsplit = cdiv(Lk, split_keys);
    const size_t part_bytes = decode_part_bytes(B, Hq, nsplit, d);
    const size_t tile_bytes = seeded ? decode_tile_bytes(B, Hq, nsplit, d, split_keys) : 0;
    const size_t need = part_bytes + tile_bytes;
    if (use_scratch) {
        if (need > size_t(MALA_DECODE_NOALLOC_SCRATCH_BYTES))
            return fail(MALA_ERR_UNSUPPORTED,
                        "split partials need %zu bytes, more than the %zu-byte static scratch (B*Hq*ceil(Lk/"
                        "split_keys)*(d+2)*4 bytes must fit)",
                        need, size_t(MALA_DECODE_NOALLOC_SCRATCH_BYTES));
        float* sp = nullptr;
        const mala_status st = scratch_of_current_device(&sp);
        if (st) return st;
        workspace = sp;
        workspace_bytes = MALA_DECODE_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need)
        return fail(MALA_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(MALA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    mala::DecArgs a{};
    a.q = q; a.kc = kcache; a.vc = vcache; a.o = o; a.lse = lse;
    a.part = static_cast<float*>(workspace);
    a.tpart = tile_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + part_bytes) : nullptr;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.Lk = Lk; a.Lcap = Lcap; a.d = d;
    a.split_keys = split_keys; a.bk = bk;
    // plain: ceil(Lk/split) partitions from key 0; seeded: ceil(ntiles/tps) partitions counted back from
    // the newest tile -- the same number, since split_keys is a multiple of bk
    a.nsplit = int(cdiv(Lk, split_keys));
    a.tps = split_keys / bk;
    a.words = int(cdiv(a.tps, 32));
    a.seeded = seeded;
    a.rpv = rows_per_vote;
    const float sc = eff_scale(scale, d);
    a.scale_log2 = sc * mala::kLog2e;
    a.log2_tau = log2_tau_of(tau);
    a.log2_lq = log2f(float(Lk));
    a.gated = tau != 0.f;
    if (stats) { a.kept = stats->kept; a.legal = stats->legal; a.bits = stats->keep_bits; a.tstat = stats->test_stat; }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipEvent_t e0 = stats ? (hipEvent_t)stats->events[0] : nullptr, e1 = stats ? (hipEvent_t)stats->events[1] : nullptr;
    hipError_t e = mala::mark(e0, s);
    if (e == hipSuccess) e = mala::launch_decode_bf16(a, s);
    if (e == hipSuccess) e = mala::mark(e1, s);
    return hip_status(e, name);
}

mala_status mala_decode(const void* q, const void* kcache, const void* vcache, int B, int Hq, int Hkv, int Lk,
                        int Lcap, int d, mala_dtype dtype, float tau, int split_keys, int bk, int rows_per_vote,
                        float scale, void* o, float* lse, mala_stats* stats, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return decode_call("mala_decode launch", false, q, kcache, vcache, B, Hq, Hkv, Lk, Lcap, d, dtype, tau,
                       split_keys, bk, rows_per_vote, scale, o, lse, stats, workspace, workspace_bytes, stream);
}

mala_status mala_decode_noalloc(const void* q, const void* kcache, const void* vcache, int B, int Hq, int Hkv,
                                int Lk, int Lcap, int d, mala_dtype dtype, float tau, int split_keys, int bk,
                                int rows_per_vote, float scale, void* o, float* lse, mala_stats* stats,
                                void* stream) {
    return decode_call("mala_decode_noalloc launch", false, q, kcache, vcache, B, Hq, Hkv, Lk, Lcap, d, dtype, tau,
                       split_keys, bk, rows_per_vote, scale, o, lse, stats, nullptr, 0, stream, true);
}

mala_status mala_decode_seeded(const void* q, const void* kcache, const void* vcache, int B, int Hq, int Hkv,
                               int Lk, int Lcap, int d, mala_dtype dtype, float tau, int split_keys, int bk,
                               int rows_per_vote, float scale, void* o, float* lse, mala_stats* stats,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return decode_call("mala_decode_seeded launch", true, q, kcache, vcache, B, Hq, Hkv, Lk, Lcap, d, dtype, tau,
                       split_keys, bk, rows_per_vote, scale, o, lse, stats, workspace, workspace_bytes, stream);
}

}  // extern "C"
