// Device-side building blocks for gfx950 (CDNA4, wave64): vector types, the
// 32x32x16 (16-bit) and 32x32x64 (E4M3) MFMAs, conversions, buffer loads and
// direct-to-LDS copies, and cross-lane exchanges.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fa355 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage element traits: 8-wide operand vector and conversions.
template <typename T> struct Vec;
template <> struct Vec<_Float16> {
    using v8 = f16x8;
    using v2 = f16x2;
};
template <> struct Vec<__bf16> {
    using v8 = bf16x8;
    using v2 = bf16x2;
};

// D(32x32, fp32) += A(32x16) * B(16x32).  Lane l supplies row (A) or column (B)
// l % 32 and eight consecutive k-slots chosen by l / 32; it receives column
// l % 32 of D, rows 8*(e/4) + 4*(l/32) + e%4 for accumulator element e.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l supplies row (A) or column
// (B) l % 16 and eight k-slots chosen by l / 16, the same way for A and B; it
// receives column l % 16 of D, rows 4 (l / 16) .. + 3.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// FP8 operands: 32 E4M3 bytes per lane.
typedef int i32x8 __attribute__((ext_vector_type(8)));

// D(32x32, fp32) += A(32x64) * B(64x32) on OCP E4M3 operands.  Lane l supplies
// row (A) or column (B) l % 32 and 32 k-slots chosen by l / 32, byte j of its
// 8 words being k-slot j of its half, the same way for A and B; D as for
// mfma32.
__device__ __forceinline__ f32x16 mfma32_e4m3(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16, fp32) += A(16x128) * B(128x16) on OCP E4M3 operands.  Lane
// l = 16 g + i supplies row (A) or column (B) i and the 32 k-slots of group g,
// byte j of its 8 words being k-slot j of the group, the same way for A and
// B; D as for mfma16.
__device__ __forceinline__ f32x4 mfma16_e4m3(i32x8 a, i32x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// fp32 -> E4M3 (OCP): nearest, ties to even; magnitudes beyond the largest
// finite value 448 (infinities included) saturate; NaN stays NaN.  Four
// values into one word, the first in the low byte.
__device__ __forceinline__ float sat448(float x) { return x != x ? x : __builtin_amdgcn_fmed3f(x, 448.f, -448.f); }
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0u, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
}

template <typename V> __device__ __forceinline__ V as(u32x4 x) { return __builtin_bit_cast(V, x); }

// Round-to-nearest-even conversions of fp32 pairs to the storage type,
// returned as one packed 32-bit word (low half = first value).
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b)
{
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b)
{
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// acc + the low / high binary16 element of w, widened exactly (one
// v_fma_mix_f32 with a 1.0 multiplier; a plain VALU instruction, unlike the
// packed dot products, which share the matrix pipeline).
__device__ __forceinline__ float add_lo_f16(float acc, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(acc));
    return r;
}
__device__ __forceinline__ float add_hi_f16(float acc, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(acc));
    return r;
}

// Widen the low / high 16-bit element of a packed word to fp32 (exact).
template <typename T> __device__ __forceinline__ float lo_f32(uint32_t w);
template <typename T> __device__ __forceinline__ float hi_f32(uint32_t w);
template <> __device__ __forceinline__ float lo_f32<_Float16>(uint32_t w)
{
    return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <> __device__ __forceinline__ float hi_f32<_Float16>(uint32_t w)
{
    return (float)__builtin_bit_cast(f16x2, w)[1];
}
template <> __device__ __forceinline__ float lo_f32<__bf16>(uint32_t w)
{
    return __builtin_bit_cast(float, w << 16);
}
template <> __device__ __forceinline__ float hi_f32<__bf16>(uint32_t w)
{
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2c_f32_{f16,bf16}).
template <typename T> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc);
template <> __device__ __forceinline__ float dot2<_Float16>(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
}
template <> __device__ __forceinline__ float dot2<__bf16>(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// Buffer resource over [base, base + bytes) (raw, stride 0).  Buffer
// accesses are range-checked against `bytes`: reads past the end return 0
// and touch no memory.  Limited to 2^32 - 1 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer resource as four scalar words: base address, stride 0, byte range
// and the same format word make_rsrc uses.  Every argument must be
// wave-uniform.
__device__ __forceinline__ u32x4 make_rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Buffer -> LDS copy of 16 bytes per lane, issued so that the compiler does
// not track it: lane i's 16 bytes from byte offset voff + soff + IMM land at
// lds_base + IMM + 16 * i (the instruction offset moves both addresses);
// reads past the range write zeros.  The compiler would otherwise make every
// later LDS read wait for the copy (it cannot tell which LDS bytes the copy
// writes), which serialises a prefetch ring.  The caller waits with
// wait_vmcnt<N>() before a barrier that publishes the data.  The LDS offset
// of a shared-memory pointer is the low 32 bits of its flat address (the
// aperture is 4 GiB aligned).
//
// The compiler does not look inside the asm for hazards, so the asm pads for
// them itself: an SGPR operand (the descriptor, the offset or M0) may have
// just been written by a VALU instruction -- for instance reloaded with
// v_readlane from a spill lane -- and a VMEM read of an SGPR written by VALU
// needs 5 wait states (s_nop 4).
template <int IMM = 0>
__device__ __forceinline__ void dma_to_lds16(u32x4 rsrc, uint32_t voff, uint32_t soff, const void *lds_base)
{
    static_assert(IMM >= 0 && IMM < 4096, "12-bit instruction offset");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%4 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "{m0}"(m0), "n"(IMM)
                 : "memory");
}

// As dma_to_lds16 with 4 bytes per lane: lane i's dword lands at
// lds_base + IMM + 4 * i.
template <int IMM = 0>
__device__ __forceinline__ void dma_to_lds4(u32x4 rsrc, uint32_t voff, uint32_t soff, const void *lds_base)
{
    static_assert(IMM >= 0 && IMM < 4096, "12-bit instruction offset");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen offset:%4 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "{m0}"(m0), "n"(IMM)
                 : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// 16-byte buffer load into registers (zeros when out of range).
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// output lane i, element j (16-bit) is element i % 4 of the 8 bytes addressed
// by lane 4 j + i / 4 of the group.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const void *lds_ptr)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)lds_ptr);
    return __builtin_bit_cast(u32x2, v);
}

// 2^x on the transcendental unit (v_exp_f32); exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// {x of this lane, x of lane ^ 32} in some order (v_permlane32_swap moves
// lanes 32..63 of its first operand and lanes 0..31 of its second across the
// halves).  Any symmetric combination (max, sum) of the pair is the same in
// both lanes.  The two results are copied to scalars before the bit cast:
// clang lowers __builtin_bit_cast of a vector element as a read of element 0.
__device__ __forceinline__ void pair_with_other_half(float x, float &a, float &b)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_with_other_half(float x)
{
    float a, b;
    pair_with_other_half(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float sum_with_other_half(float x)
{
    float a, b;
    pair_with_other_half(x, a, b);
    return a + b;
}

// DPP lane exchanges inside a 16-lane row.
enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141, // lane i <-> 7 - i within each half row
    kDppMirror = 0x140      // lane i <-> 15 - i within the row
};
template <int CTRL> __device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of the group gets the sum.
template <int N> __device__ __forceinline__ float group_sum(float x)
{
    static_assert(N == 8 || N == 16, "group size");
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    if constexpr (N == 16) x += dpp<kDppMirror>(x);
    return x;
}

// Debug builds (-DFA355_POISON_LDS): every kernel fills its LDS arrays with
// all-ones words before their first use.  0xFFFFFFFF is a NaN as fp32, as
// each fp16 or bf16 half and as each E4M3 byte, so a read of LDS that the
// kernel never wrote, if it reaches an output, turns that output into NaN
// and the parity tests reject it.  Normal builds compile none of this.
#ifdef FA355_POISON_LDS
constexpr bool kPoisonLds = true;
#else
constexpr bool kPoisonLds = false;
#endif
__device__ __forceinline__ void poison_lds(void *p, unsigned bytes)
{
    unsigned *w = static_cast<unsigned *>(p);
    for (unsigned i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = ~0u;
}

}  // namespace fa355
