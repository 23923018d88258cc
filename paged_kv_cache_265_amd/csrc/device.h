// device.h -- element types, conversions and CDNA4 matrix-core wrappers shared by
// the gfx950 kernels of this library.  Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Element kinds.  Storage is always raw bits; arithmetic is fp32.
enum Kind { KF32 = 0, KF16 = 1, KBF16 = 2 };

template <int K> struct Elem;
template <> struct Elem<KF32> { typedef float bits; static constexpr int bytes = 4; };
template <> struct Elem<KF16> { typedef uint16_t bits; static constexpr int bytes = 2; };
template <> struct Elem<KBF16> { typedef uint16_t bits; static constexpr int bytes = 2; };

// ---- conversions -------------------------------------------------------------------

// low / high 16-bit half of a 32-bit word, widened to fp32
template <int K> __device__ __forceinline__ float lo16(uint32_t w);
template <int K> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<KBF16>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float hi16<KBF16>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo16<KF16>(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <> __device__ __forceinline__ float hi16<KF16>(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2, w)[1];
}

// fp32 -> storage bits, round to nearest even (hardware conversions on gfx950)
template <int K> __device__ __forceinline__ uint16_t to_bits16(float x);
template <> __device__ __forceinline__ uint16_t to_bits16<KBF16>(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ uint16_t to_bits16<KF16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int K> __device__ __forceinline__ void store_elem(void* base, size_t i, float x) {
    if constexpr (K == KF32)
        ((float*)base)[i] = x;
    else
        ((uint16_t*)base)[i] = to_bits16<K>(x);
}

// Two fp32 values -> two 16-bit values in one word (a in the low half), round to
// nearest even: one two-source conversion instruction on gfx950.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int K> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<KBF16>(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<KF16>(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// Four fp32 values -> four 16-bit values packed in 8 bytes.
template <int K> __device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack2<K>(a, b), pack2<K>(c, d));
}

// ---- matrix cores --------------------------------------------------------------------
// 16x16x32 (A: 16 rows x 32 k, 8 elements per lane; lane l holds row l%16,
// k = 8*(l/16)..+7; B symmetric with columns) and 16x16x16 (4 elements per lane,
// k = 4*(l/16)..+3).  Result: lane l holds rows 4*(l/16)..+3 of column l%16.
template <int K> __device__ __forceinline__ f32x4 mma_16x16x32(uint4 a, uint4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mma_16x16x32<KBF16>(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma_16x16x32<KF16>(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}
template <int K> __device__ __forceinline__ f32x4 mma_16x16x16(uint2 a, uint2 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mma_16x16x16<KBF16>(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                     0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma_16x16x16<KF16>(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                 0, 0);
}

// 32x32x16 (A: 32 rows x 16 k, 8 elements per lane; lane l holds row l%32,
// k = 8*(l/32)..+7; B symmetric with columns).  Result: lane l holds column
// l%32, rows 8*(r/4) + 4*(l/32) + r%4 in element r (r = 0..15).
template <int K> __device__ __forceinline__ f32x16 mma_32x32x16(uint4 a, uint4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mma_32x32x16<KBF16>(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mma_32x32x16<KF16>(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

// Lanes of rows 0 and 2 (16-lane rows) keep their own value in `a` and receive
// row 1 / row 3's value of `x` in `b`; lanes of rows 1 and 3 receive row 0 / row
// 2's value of `y` in `a` and keep their own `y` in `b` (v_permlane16_swap).
__device__ __forceinline__ void row_swap16(uint32_t x, uint32_t y, uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    a = r[0];
    b = r[1];
}

// ---- streaming loads -----------------------------------------------------------------
// K/V tiles are read exactly once per call: load them with the non-temporal hint
// so they do not displace reused data in the caches.
__device__ __forceinline__ uint4 stream_load16(const void* p) {
    const u32x4 x = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 stream_load8(const void* p) {
    const u32x2 x = __builtin_nontemporal_load((const u32x2*)p);
    return make_uint2(x.x, x.y);
}

// Buffer resource over the `bytes` bytes at `base` (raw, unswizzled; dword 3 as
// the gfx9 family takes it).  Loads at offsets past `bytes` return zeros and make
// no memory access, so a pipeline can issue a load on every iteration -- with
// bytes = 0 once it has run out of tiles -- and the compiler can count exactly
// which of its loads are still in flight.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// `base` and `bytes` must be wave-uniform; they are taken from the first lane so
// that the resource sits in scalar registers.
__device__ __forceinline__ rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), 0, __builtin_amdgcn_readfirstlane((int)bytes),
                                             0x00020000);
}
constexpr int kNonTemporal = 2;  // cache-policy bit of the buffer loads: nt
__device__ __forceinline__ uint4 stream_load16(rsrc_t r, uint32_t off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 stream_load8(rsrc_t r, uint32_t off) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kNonTemporal);
    return make_uint2(x.x, x.y);
}
// The same with a choice of cache policy: kAux = kNonTemporal streams, 0 keeps the
// default policy (for lines whose other half another load reads soon after).
template <int kAux> __device__ __forceinline__ uint4 policy_load16(rsrc_t r, uint32_t off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAux);
    return make_uint4(x.x, x.y, x.z, x.w);
}
template <int kAux> __device__ __forceinline__ uint2 policy_load8(rsrc_t r, uint32_t off) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kAux);
    return make_uint2(x.x, x.y);
}

// Fence between a chain of 16x16x32 matrix-core products and the first vector-ALU
// read of its result.  A 4-pass XDL product writing VGPRs must be followed by 8 wait
// states before a VALU instruction reads the result on gfx950 (the compiler pads the
// fall-through path with exactly that many).  Where the read sits at the head of a
// block reached by a taken branch -- the softmax's unmasked path, jumped to right after
// the score products -- this compiler inserts none: the read followed the product by a
// single wait state, and outputs differed in their last bits from run to run.  Eight
// wait states here, with nothing scheduled across them, cover every path.
__device__ __forceinline__ void mfma_result_fence() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// ---- misc ------------------------------------------------------------------------------

// True when the call's contract pre-pass found a violation (see Guard): the kernel
// then does nothing.  A NULL guard (checks off) costs one test of a kernel argument.
__device__ __forceinline__ bool contract_broken(const unsigned long long* guard) {
    return guard && *(const volatile unsigned long long*)guard != ~0ull;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): for operands that are never NaN it
// equals fmaxf, without the operand quieting fmaxf needs in IEEE mode
__device__ __forceinline__ float max_nonan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Assert that v is the same in every lane, so that addresses built from it stay in
// scalar registers: loads through them are then scalar loads, which the wave waits
// for separately from its vector loads still in flight.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform(long long v) {
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (long long)(lo | (hi << 32));
}

// Wait until every vector memory access of this wave has completed (s_waitcnt
// vmcnt(0); the expcnt and lgkmcnt fields are left at their maximum).  Placed
// right after loads made on a rarely taken path, it keeps the compiler from
// waiting for them -- and with them for everything issued before -- on every
// path that joins afterwards.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N vector memory accesses of this wave are outstanding
// (vmcnt is six bits: [3:0] and [15:14] of the immediate).
template <int N> __device__ __forceinline__ void vm_wait_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

// Scalar load of base[i] with a wave-uniform i, for tables the kernel only reads
// (block tables, context lengths): through the constant address space the compiler
// may use the scalar cache even though the kernel stores elsewhere.
__device__ __forceinline__ int scalar_load(const int32_t* base, size_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)base)[i];
}

// the same for a 64-bit value stored as two 32-bit words, low word first
__device__ __forceinline__ long long scalar_load64(const int32_t* base, size_t i) {
    const uint32_t lo = (uint32_t)scalar_load(base, i), hi = (uint32_t)scalar_load(base, i + 1);
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// value of a wave-uniform register from lane `src` (src must be wave-uniform)
__device__ __forceinline__ int read_lane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float read_lane(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// v and the value of lane (lane ^ 16) or (lane ^ 32), as a pair: gfx950's row swaps
// exchange rows 0<->1 and 2<->3 (16-lane rows) or the two 32-lane halves in one
// vector instruction, without the LDS round trip of a general lane permute.  With
// both operands equal to v, every lane ends up holding its own value in one result
// and its partner's in the other.
__device__ __forceinline__ void swap_pair(float v, int mask, float& a, float& b) {
    const uint32_t u = __float_as_uint(v);
    if (mask == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    }
}

__device__ __forceinline__ float xor_max(float v, int mask) {
    if (mask == 16 || mask == 32) {
        float a, b;
        swap_pair(v, mask, a, b);
        return fmaxf(a, b);
    }
    return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
    if (mask == 16 || mask == 32) {
        float a, b;
        swap_pair(v, mask, a, b);
        return a + b;
    }
    return v + __shfl_xor(v, mask, 64);
}

constexpr float kLog2e = 1.4426950408889634f;
// Online softmax with a lazy reference: probabilities are 2^(x - m) with x the
// scaled score and m a reference that is raised (and the running sums rescaled)
// only when some row's maximum exceeds it by more than this many powers of two.
// In between, probabilities stay below 2^8 -- far inside fp32 (and 16-bit) range
// -- and the common case skips the rescale entirely.
constexpr float kRescaleSlack = 8.f;
constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace pkv
