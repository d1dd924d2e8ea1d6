// MFMA building blocks shared by the 16-bit attention kernels (gfx950):
// element traits for bf16 / f16 operands, the LDS swizzles, HBM -> LDS tile
// DMA, LDS operand reads issued through asm with explicit lgkmcnt waits, and
// the half-wave exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {
namespace mfma {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16-bit storage types: the operand vectors, the 32x32x16 MFMA and the
// paired dot product used for row sums.  f16 and bf16 operands have the
// same register layout, so the kernel is one template over them.
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
    }
};
template <>
struct Elem<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS position (in 16-byte chunks within the row) of chunk c of K row r, and
// of chunk q of V row r.  gfx950 serves 16 lanes of a 128-bit read per
// cycle from 64 banks (256 bytes), so the 16 rows GEMM0 reads together must
// fall into 16 different 16-byte bank groups.  With KCH = 8 (mod 16) rows
// start alternately at group 0 and 8, and c ^ ((r >> 1) & 7) spreads each
// pair over the other 8 groups; with KCH = 0 (mod 16), c ^ (r & 15).  V: the
// transpose reads take 64 bytes of 4 consecutive rows; 4 (r % 4) moves each
// of those rows to its own quarter of the banks.
template <int KCH>
__device__ __forceinline__ int k_swz(int r, int c) {
    if constexpr (KCH % 16 == 0) return c ^ (r & 15);
    else return c ^ ((r >> 1) & 7);
}
template <int VG>
__device__ __forceinline__ int v_swz(int r, int q) { return q ^ (4 * (r % VG)); }

// Buffer resource over [base, base + bytes): loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc + voffset into LDS at lds_wave_base + 16 * lane.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint16_t* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, voffset, 0, 0, 0);
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane i receives
// element i % 4 of the 8-byte rows addressed by lanes 4j + i / 4, j = 0..3.
// Issued through asm so that the compiler does not hold it behind the
// in-flight HBM -> LDS tile loads (they write the other buffer); the caller
// waits on lgkmcnt explicitly before using the result (tr_wait).
template <int OFS>
__device__ __forceinline__ s16x4 tr_read(uint32_t addr) {
    s16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFS));
    return r;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// ds_read_b128 through asm, for the same reason as tr_read (GEMM0's K
// fragments are read one step ahead of the MFMAs that use them).
template <int OFS>
__device__ __forceinline__ i32x4_t k_read(uint32_t addr) {
    i32x4_t r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFS));
    return r;
}

template <int N>
__device__ __forceinline__ void k_wait(i32x4_t& a, i32x4_t& b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// Value of lane l ^ 32 (the other half-wave).  v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second, so
// with both = x the first result holds x[l - 32] in lanes 32..63 and the
// second holds x[l + 32] in lanes 0..31.
__device__ __forceinline__ float other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Waits until at most N LDS reads are outstanding; the operands tie the wait
// to the registers those reads fill, so no use can be scheduled before it.
template <int N>
__device__ __forceinline__ void tr_wait(s16x4 (&x)[8]) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
                 : "i"(N));
}

}  // namespace mfma
}  // namespace sk
