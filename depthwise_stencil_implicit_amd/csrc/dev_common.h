// Device-side helpers shared by the gfx950 kernels: storage types, exact
// widening to fp32, round-to-nearest-even narrowing, and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miconv {

// Storage types: the kernels move raw bits and convert explicitly.
struct bf16_t { uint16_t u; };
struct f16_t { uint16_t u; };

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

template <typename T> struct Dt;
template <> struct Dt<float> {
    static constexpr int size = 4;
    static constexpr int code = 0;
};
template <> struct Dt<f16_t> {
    static constexpr int size = 2;
    static constexpr int code = 1;
};
template <> struct Dt<bf16_t> {
    static constexpr int size = 2;
    static constexpr int code = 2;
};

// Widen one element to fp32 (exact for every input type).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.u << 16); }
__device__ __forceinline__ float to_f32(f16_t v)
{
    _Float16 h;
    __builtin_memcpy(&h, &v.u, 2);
    return (float)h;
}

// Low / high 16-bit halves of a packed word, widened.
__device__ __forceinline__ float lo_f32(uint32_t w, bf16_t) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w, bf16_t) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float lo_f32(uint32_t w, f16_t) { return to_f32(f16_t{(uint16_t)(w & 0xffffu)}); }
__device__ __forceinline__ float hi_f32(uint32_t w, f16_t) { return to_f32(f16_t{(uint16_t)(w >> 16)}); }

// Two products of a packed 16-bit pair added to an fp32 accumulator:
// c + a.lo*b.lo + a.hi*b.hi (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <typename T> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <> __device__ __forceinline__ float dot2<f16_t>(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}
template <> __device__ __forceinline__ float dot2<bf16_t>(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// The same sum written to a fresh register: the VOP3P encoding, whose
// accumulator input is an operand of its own.  The compiler always picks the
// tied v_dot2c form and, for an accumulator that stays live (a bias starting
// several chains), first copies it into the destination; this form needs no
// copy.  Bit-identical to dot2 (compared on 2^20 random bf16 operand sets).
template <typename T> __device__ __forceinline__ float dot2_to(uint32_t a, uint32_t b, float c);
template <> __device__ __forceinline__ float dot2_to<f16_t>(uint32_t a, uint32_t b, float c)
{
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
template <> __device__ __forceinline__ float dot2_to<bf16_t>(uint32_t a, uint32_t b, float c)
{
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Narrow fp32 to the storage type, rounding to nearest even.
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v)
{
    __bf16 h = (__bf16)v;
    bf16_t r;
    __builtin_memcpy(&r.u, &h, 2);
    return r;
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v)
{
    _Float16 h = (_Float16)v;
    f16_t r;
    __builtin_memcpy(&r.u, &h, 2);
    return r;
}

// Narrow two fp32 values into one packed 32-bit word (lo, hi), each rounded
// to nearest even: one vector conversion (a single v_cvt_pk_bf16_f32 for
// bf16).
typedef __attribute__((ext_vector_type(2))) float f32x2;
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

template <typename T> __device__ __forceinline__ T load_elem(const T *p) { return *p; }

// Raw buffer descriptor (the same fields __builtin_amdgcn_make_buffer_rsrc
// fills: base, stride 0, byte range, the flags word) as an SGPR quad for
// inline assembly.
__device__ __forceinline__ u32x4 raw_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}
// 16-byte raw buffer store followed by two wait states.  The hardware may
// still be reading the data registers of a store wider than 8 bytes when the
// next instruction issues, and a VALU write to them in that cycle changes
// what is stored (seen on gfx950: the next store's address landed in the
// first word of the previous one's data, and the compiler did not pad the
// pair).  In one asm block nothing can be scheduled between the two.
// Stores of whole output lines are non-temporal (nt): a kernel never reads
// back what it writes, and streaming those lines out of the L2 measured 6-11%
// faster on the depthwise and grouped kernels.  (Stores of partial lines --
// the implicit GEMM's 8-byte pieces -- keep the default policy: there the L2
// merges the pieces, and nt measured 11-15% slower.)
constexpr int kStoreNT = 2;   // cache-policy operand of the buffer-store builtins: nt
__device__ __forceinline__ void store_b128(u32x4 v, u32x4 rsrc, int voff, int soff)
{
    asm volatile("buffer_store_dwordx4 %0, %1, %2, %3 offen nt\n\ts_nop 1" ::"v"(v), "v"(voff), "s"(rsrc),
                 "s"(soff)
                 : "memory");
}

// 8-element MFMA step: D(16x16) += A(16x32) * B(32x16) for 2-byte types, with
// the A/B fragments holding 8 consecutive K elements of one row / column.
__device__ __forceinline__ void mma_16x16x32(const uint4 &a, const uint4 &b, f32x4 &c, bf16_t)
{
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}
__device__ __forceinline__ void mma_16x16x32(const uint4 &a, const uint4 &b, f32x4 &c, f16_t)
{
    f16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

// fp32: eight 16x16x4 steps cover the same 32-wide K slice.  Lane l's j-th
// element is K index 8*(l/16) + j; step j feeds element j of every lane, so
// step j sums K = {j, 8+j, 16+j, 24+j}: together the eight steps sum all 32.
__device__ __forceinline__ void mma_16x16x32_f32(const float (&a)[8], const float (&b)[8], f32x4 &c)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

// Workgroups are dealt to the 8 XCDs round-robin; block b is remapped so
// that each XCD gets one contiguous range of tiles (tiles that share input
// rows or weight slices then share that XCD's L2).
__device__ __forceinline__ int xcd_tile(int b, int total)
{
    const int q = total >> 3, r = total & 7;
    const int xcd = b & 7, local = b >> 3;
    const int off = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return off + local;
}

// A workgroup barrier without a memory fence: a compiler-only memory
// clobber keeps LDS accesses on their side of it.  Before it each wave waits
// for its own direct-to-LDS loads of the stage about to be read, so after it
// every wave's loads have landed; a fenced __syncthreads() would instead
// drain every load in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Byte offset of 16-byte chunk c of LDS row r with KC chunks per row.  KC = 8:
// c ^ (r & 7); KC = 4: c ^ ((r >> 1) & 3).  Either way the 8 lanes of one
// ds_read_b128 cycle (8 consecutive rows, one logical chunk) land on 8
// different 16-byte bank groups.
template <int KC> __device__ __forceinline__ int swz_k(int r, int c)
{
    if constexpr (KC == 8) return (r * 8 + (c ^ (r & 7))) * 16;
    else return (r * 4 + (c ^ ((r >> 1) & 3))) * 16;
}

}  // namespace miconv
