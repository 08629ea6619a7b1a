// Device helpers shared by the MALA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mala {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// compute units of a gfx950 GPU (MI350X / MI355X: 8 XCDs x 32 CUs); launchers size grids against it
constexpr int kNumCUs = 256;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return bf16_t(pack_bf16x2(f, 0.f) & 0xffffu); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 32x32x16 bf16 MFMA: D[i][j] = C[i][j] + sum_k A[i][k] B[k][j].
// Lane l holds A[l%32][8*(l/32) .. +8], B[8*(l/32) .. +8][l%32];
// D register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// 16x16x32 bf16 MFMA: D[i][j] = C[i][j] + sum_k A[i][k] B[k][j].
// Lane l holds A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16];
// D register r of lane l is D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Work item of workgroup i in a grid ordered by rank (i / BH) and head.  The
// GPU deals workgroups to its 8 XCDs round-robin (i % 8), so with head =
// i % BH every XCD would serve a fixed subset of the heads for the whole
// launch, and an XCD whose heads skip most tiles would idle while the others
// finish.  Rotating the head by one every `period` ranks (the shift is one
// constant per rank, so each rank still covers every head once) moves every
// XCD through all heads, while workgroups that run together on an XCD still
// share a head and its L2 lines.
__device__ __forceinline__ void balanced_item(int i, int BH, int period, int& rank, int& head) {
    rank = i / BH;
    head = (i - rank * BH + rank / period) % BH;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

// x combined with the value of lane i^32, in every lane: op(x[i % 32], x[i % 32 + 32]).
// v_permlane32_swap with both operands x leaves the low half in the first
// result and the high half in the second, so no LDS traffic is involved; the
// operations are commutative, so every lane gets the xor-32 butterfly's value.
__device__ __forceinline__ float max_halves(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global loads (vmcnt), so direct global->LDS prefetches stay in flight across
// it.  The memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- LDS tiles
// Tiles of 128-element bf16 rows (256 B per row) are kept row-major in LDS
// with their 16-byte chunks XOR-swizzled by a permutation of the row's low 4
// bits (the two 2-bit fields swapped).  Conflict-free for both patterns used:
// 16 consecutive rows at one chunk (MFMA operand reads, tile stores) hit 16
// distinct chunks, and the transposed reads below -- 8 consecutive rows x 4
// consecutive chunks -- hit every chunk exactly twice.
__device__ __forceinline__ int rowkey(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ rowkey(row)) << 4); }
__device__ __forceinline__ int swz_el(int row, int d) { return swz(row, d >> 3) + ((d & 7) << 1); }

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b64_tr_b16: within each 16-lane group the lanes read a 16x4 block
// M of 16-bit elements (one 8-byte row per lane) and lane i receives
// M[i/4 + 4e][i%4], e = 0..3.
__device__ __forceinline__ u32x2 tr16(const uint8_t* lds_base, int byte_off) {
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    lds_bf16x4* p = (lds_bf16x4*)((lds_u8*)const_cast<uint8_t*>(lds_base) + byte_off);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p));
}

// LDS pointer from a 32-bit LDS byte address.
__device__ __forceinline__ const uint8_t* lds_ptr(uint32_t addr) {
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    return (const uint8_t*)(lds_u8*)(uintptr_t)addr;
}

// Per-lane byte offsets of the transposed operand reads of tr_operand within
// a tile (rowbase 0): [db][0] for rows 4hl + {0..3}, [db][1] for rows
// 8 + 4hl + {0..3}.  Adding 256*rowbase (rowbase a multiple of 16) gives the
// offsets for other row bases, because the swizzle depends on row % 16 only.
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[4][2]) {
    const int g = lane >> 4, i = lane & 15, a = i & 3, es = i >> 2;
    const int hl = g >> 1, dh = g & 1;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + 16 * dh + 4 * a;
        off[db][0] = swz_el(4 * hl + es, d);
        off[db][1] = swz_el(8 + 4 * hl + es, d);
    }
}

// tr_operand with precomputed offsets: base = LDS address of the tile plus
// 256 * rowbase.
__device__ __forceinline__ u32x4 tr_operand_at(uint32_t base, const int (&off)[2]) {
    const u32x2 lo = tr16(lds_ptr(base), off[0]);
    const u32x2 hi = tr16(lds_ptr(base), off[1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// A operand of a 32x32x16 product whose contraction runs over the ROWS of a
// swizzled tile: lane l gets column d = 32*db + l%32 at rows
// rowbase + 4*(l/32) + {0..3} and rowbase + 8 + 4*(l/32) + {0..3} -- the row
// order of registers 8*hf .. 8*hf+7 of a 32x32 accumulator block.
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* tile, int rowbase, int db, int lane) {
    const int g = lane >> 4, i = lane & 15, a = i & 3, es = i >> 2;
    const int hl = g >> 1, dh = g & 1;
    const int d = 32 * db + 16 * dh + 4 * a;
    const int r = rowbase + 4 * hl + es;
    const u32x2 lo = tr16(tile, swz_el(r, d));
    const u32x2 hi = tr16(tile, swz_el(r + 8, d));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// One direct global->LDS load: every lane reads 16 bytes at sbase + voff;
// lane l's bytes land at LDS byte address lds_addr + 16*l (lds_addr must be
// the same in all lanes).  The data goes to LDS, not to registers, and
// completion is tracked by the callers with explicit s_waitcnt vmcnt(N)
// before the barrier that publishes the tile.  Written as asm rather than
// with __builtin_amdgcn_global_load_lds because the compiler cannot tell
// which LDS bytes such a load writes and then waits for every outstanding
// load before each later LDS access, which would serialize the prefetch.  The
// asm has no register outputs (nothing can be overwritten late); it clobbers
// M0.  The saddr form takes a wave-uniform 64-bit base in SGPRs and a
// per-lane 32-bit byte offset: one VGPR of address per lane instead of two.
// The base must be the same in every lane; it is read from the first lane
// so that it always sits in an SGPR pair.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    // (the builtin returns a signed int: both halves go through uint32_t so
    // that the low half is zero-extended, never sign-extended)
    const uint64_t b = reinterpret_cast<uint64_t>(sbase);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b))));
    const uint32_t hi =
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32))));
    const void* sb = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo));
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(lds_addr)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((lds_void*)const_cast<void*>(p)));
}

}  // namespace mala
