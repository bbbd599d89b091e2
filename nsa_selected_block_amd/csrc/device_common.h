// device_common.h -- device helpers shared by the forward and backward
// kernels: 16-bit element types (bf16, fp16) with their conversions and MFMA,
// work-item decoding and the staging of a kv block (K rows, V transposed)
// into LDS.
#pragma once

#include "internal.h"

namespace nsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float bf16_to_f32(u16 x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ u16 f32_to_bf16(float x)
{
    __bf16 b = static_cast<__bf16>(x);  // round to nearest even
    return __builtin_bit_cast(u16, b);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// 16-bit element types of the MFMA kernels.  Inputs and outputs are either
// bf16 or fp16; accumulation is fp32 either way.
template <typename E> struct H16;

template <> struct H16<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ float to_f32(u16 x) { return __uint_as_float((uint32_t)x << 16); }
    static __device__ __forceinline__ u16 bits(float x)  // round to nearest even
    {
        const __bf16 b = static_cast<__bf16>(x);
        return __builtin_bit_cast(u16, b);
    }
    static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct H16<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ float to_f32(u16 x) { return (float)__builtin_bit_cast(_Float16, x); }
    static __device__ __forceinline__ u16 bits(float x)  // round to nearest even
    {
        const _Float16 h = static_cast<_Float16>(x);
        return __builtin_bit_cast(u16, h);
    }
    static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Two floats rounded to E and packed low, high.
template <typename E>
__device__ __forceinline__ uint32_t pack2h(float lo, float hi)
{
    return (uint32_t)H16<E>::bits(lo) | ((uint32_t)H16<E>::bits(hi) << 16);
}

// Four floats rounded to E (nearest even) as packed pairs, and eight as an
// MFMA operand; vector conversions map to the packed convert instructions.
template <typename E>
__device__ __forceinline__ uint2 cvt4(f32x4 v)
{
    typedef E e4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(uint2, __builtin_convertvector(v, e4));
}
template <typename E>
__device__ __forceinline__ typename H16<E>::v8 cvt8(f32x4 lo, f32x4 hi)
{
    const uint2 a = cvt4<E>(lo), b = cvt4<E>(hi);
    return __builtin_bit_cast(typename H16<E>::v8, make_uint4(a.x, a.y, b.x, b.y));
}

// Lane l's value combined with lane l ^ 32's, and with lane l ^ 16's, by the
// cross-lane swap instructions; both operands are the same on the two lanes
// of a pair, so every lane gets the bitwise same result.
__device__ __forceinline__ float xmax32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Minimum over the 16 lanes of each DPP row (lanes 16 r .. 16 r + 15), by
// four row rotations; every lane of a row gets the row's minimum.
__device__ __forceinline__ int row16_min(int x)
{
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));  // row_ror:8
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));  // row_ror:4
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xF, 0xF, false));  // row_ror:2
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xF, 0xF, false));  // row_ror:1
    return x;
}

// LDS image of a staged key block: rows of D 16-bit values, unpadded, the
// 16-byte chunks of row r XOR-permuted: K by kswz(r), so that a K operand
// read (16 rows, one chunk) meets every bank once; V by vswz(r), so that a
// transpose read of V (per 16 lanes: 4 rows, two neighbouring chunks) does.
template <int D> __device__ __forceinline__ int kswz(int r) { return r & ((D / 8 < 16 ? D / 8 : 16) - 1); }
template <int D> __device__ __forceinline__ int vswz(int r) { return (r & ((D / 8 < 16 ? D / 8 : 16) / 2 - 1)) << 1; }

// Bucket of a work item, decoded.
struct Bucket {
    int h, c0, kbeg, nkeys, off, cnt;
};

__device__ __forceinline__ Bucket decode_bucket(const Params& p, int bkt)
{
    Bucket bk;
    bk.h = bkt / p.nbc;
    const int g = bkt - bk.h * p.nbc;
    int slo = 0, shi = p.B - 1;  // last sequence with blkoff <= g
    while (slo < shi) {
        int mid = (slo + shi + 1) >> 1;
        if (p.blkoff[mid] <= g) slo = mid; else shi = mid - 1;
    }
    const int j = g - p.blkoff[slo];
    bk.c0 = p.cus[slo];
    const int L = p.cus[slo + 1] - bk.c0;
    bk.kbeg = j * p.bs;
    bk.nkeys = min(p.bs, L - bk.kbeg);
    bk.off = p.offsets[bkt];
    bk.cnt = p.offsets[bkt + 1] - bk.off;
    return bk;
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// decode_bucket with every field moved to scalar registers (the bucket is
// the same for the whole workgroup).
__device__ __forceinline__ Bucket decode_bucket_uni(const Params& p, int b)
{
    Bucket bk = decode_bucket(p, b);
    bk.h = uni(bk.h); bk.c0 = uni(bk.c0); bk.kbeg = uni(bk.kbeg);
    bk.nkeys = uni(bk.nkeys); bk.off = uni(bk.off); bk.cnt = uni(bk.cnt);
    return bk;
}

// Raw buffer resource over [base, base + bytes) (wave-uniform).  Buffer
// loads outside the range return 0 and buffer stores outside it are dropped
// by the hardware, so partial tiles need no branch around their memory
// instructions.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kBufNT = 2;                 // cache-policy bits of a non-temporal buffer access
constexpr uint32_t kBufOff = 0x40000000u; // a lane offset beyond every range used here

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Two LDS transpose reads (ds_read_b64_tr_b16) joined into one 8-element operand.
template <typename V8>
__device__ __forceinline__ V8 lds_tr_pair(const u16* a, const u16* b)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(V8, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// k-th item of XCD queue x: groups of kQueueGroup consecutive items are dealt
// round-robin over the queues.
__device__ __forceinline__ int queue_item(int k, int x)
{
    return ((k / kQueueGroup) * kNumXcd + x) * kQueueGroup + (k % kQueueGroup);
}

}  // namespace

}  // namespace nsa
