// device.h - gfx950 device helpers: element traits with packed loads/stores,
// round-to-nearest-even output conversion, and cross-lane sums built on DPP,
// ds_swizzle and v_readlane (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsn {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT> struct ElemSize { static constexpr int value = DT == DT_F32 ? 4 : 2; };

// Raw storage for VEC elements of dtype DT, loaded with one instruction:
// 16 bytes -> global_load_dwordx4, 8 -> dwordx2, 4 -> dword, 2 -> ushort.
template <int BYTES> struct RawBits;
template <> struct RawBits<16> { using type = u32x4; };
template <> struct RawBits<8> { using type = u32x2; };
template <> struct RawBits<4> { using type = uint32_t; };
template <> struct RawBits<2> { using type = uint16_t; };

template <int DT, int VEC> struct Pack {
    static constexpr int BYTES = VEC * ElemSize<DT>::value;
    using raw_t = typename RawBits<BYTES>::type;
    raw_t v;
};

// 32-bit word w of a raw pack (w < BYTES/4), or the zero-extended 16-bit
// element for 2-byte packs.
template <int DT, int VEC>
__device__ __forceinline__ uint32_t word(const Pack<DT, VEC> &p, int w) {
    if constexpr (Pack<DT, VEC>::BYTES >= 8) {
        return p.v[w];
    } else {
        return (uint32_t)p.v;
    }
}

// Element e of a pack, widened exactly to fp32.
template <int DT, int VEC>
__device__ __forceinline__ float elem(const Pack<DT, VEC> &p, int e) {
    if constexpr (DT == DT_F32) {
        return __uint_as_float(word(p, e));
    } else if constexpr (DT == DT_BF16) {
        uint32_t w = word(p, e >> 1);
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        uint32_t w = word(p, e >> 1);
        f16x2 h = __builtin_bit_cast(f16x2, w);
        return (float)h[e & 1];
    }
}

// Round two fp32 values to nearest-even in the dtype and pack them into one
// 32-bit word (lower element first): v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (DT == DT_BF16) {
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <int DT>
__device__ __forceinline__ uint16_t pack1(float a) {
    if constexpr (DT == DT_BF16) {
        return __builtin_bit_cast(uint16_t, (__bf16)a);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)a);
    }
}

// Round VEC fp32 values to the dtype (nearest-even) into a raw pack.
template <int DT, int VEC>
__device__ __forceinline__ Pack<DT, VEC> make_pack(const float (&f)[VEC]) {
    Pack<DT, VEC> p;
    if constexpr (DT == DT_F32) {
        if constexpr (VEC == 1) {
            p.v = __float_as_uint(f[0]);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) p.v[e] = __float_as_uint(f[e]);
        }
    } else if constexpr (VEC == 1) {
        p.v = pack1<DT>(f[0]);
    } else if constexpr (VEC == 2) {
        p.v = pack2<DT>(f[0], f[1]);
    } else {
#pragma unroll
        for (int w = 0; w < VEC / 2; ++w) p.v[w] = pack2<DT>(f[2 * w], f[2 * w + 1]);
    }
    return p;
}

// The value an fp32 number takes once stored in the dtype and read back.
template <int DT>
__device__ __forceinline__ float round_trip(float a) {
    if constexpr (DT == DT_F32) {
        return a;
    } else if constexpr (DT == DT_BF16) {
        return __uint_as_float((uint32_t)pack1<DT>(a) << 16);
    } else {
        return (float)(_Float16)a;
    }
}

// ---------------------------------------------------------------------------
// Buffer resources. A raw buffer descriptor (base address, byte range) lives in
// four SGPRs; loads through it whose offset lies outside the range return zero
// and stores outside it are dropped, in hardware. The kernels use that range
// check instead of branches around memory operations: a row chunk past the
// row end, or a row past the last row, gets an offset outside the range.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a gfx9-family buffer descriptor: 32-bit data format, identity
// channel selects (the value the CDNA ISA defines for raw byte buffers).
constexpr int RSRC_WORD3 = 0x00020000;
// An offset no descriptor range reaches (every range here is below 2^31).
constexpr uint32_t OOB = 0x80000000u;
// Cache-policy bits of a buffer access on gfx950 (bit 0 SC0, bit 1 NT,
// bit 4 SC1). NT marks data streamed once; SC1 marks a store system-coherent.
// The streamed row loads use NT (without it the long runs lose 7%). The
// main kernel's plain and LayerNorm backwards store their single streamed
// output, dx, with SC1 on 16-byte chunks, except on rows of 512 threads
// that hold 16 or more elements each (LayerNorm) or 32 or more 16-bit
// elements (plain); those rows, the fused-add backward, the element path
// and the long-row backwards store with NT. The
// plain and LayerNorm forwards store y with SC1 where a
// thread holds fewer than 16 elements of a row (16-bit rows of at most 4096
// elements on the vector path) and with NT where it holds more (and in the
// long-row kernels); the fused forward stores with NT.
// Measured on MI355X, bf16: SC1 takes the plain backward at 4096 x 4096
// from 23.0 to 22.2 us and at 16384 x 4096 from 69.5 to 65.5 us (against
// default stores; NT there: 4096 x 4096 20.4 -> 21.3 us, 16384 x 8192
// 121.7 -> 131-137 us against SC1), while the fused backward runs 0.7 us
// slower with it at 1024 x 8192. The plain forward's y, NT against SC1,
// depends on the row length: 1024 x 8192 7.7 -> 6.9-7.1 us, 16384 x 8192
// 91.6 -> 89.1 us, 32768 x 8192 195 -> 183 us, long rows 128 x 32768 5.9 ->
// 5.4 us, 4096 x 24576 68.9 -> 66.3 us, the element path 4096 x 4097 25.3
// -> 22.1 us; but 16384 x 4096 42.3 -> 47.5 us, 16384 x 2048 22.6 -> 25.1
// us, 32768 x 1024 22.7 -> 25.1 us and 4096 x 4096 12.8 -> 13.3 us with
// rotated buffer sets of three row arrays (sets of two arrays measured NT
// up to 3% faster there). SC1 is faster than default stores (plain 16384 x
// 4096 48 -> 42 us). All are build-time knobs.
constexpr int AUX_DEFAULT = 0;
constexpr int AUX_NT = 2;
#ifndef RMSN_LOAD_AUX
#define RMSN_LOAD_AUX 2
#endif
#ifndef RMSN_STORE_AUX
#define RMSN_STORE_AUX 2
#endif
#ifndef RMSN_SINGLE_STORE_AUX
#define RMSN_SINGLE_STORE_AUX 16
#endif
#ifndef RMSN_FWD_STORE_AUX
#define RMSN_FWD_STORE_AUX 2
#endif
#ifndef RMSN_FWD_SHORT_STORE_AUX
#define RMSN_FWD_SHORT_STORE_AUX 16
#endif
constexpr int AUX_STREAM_LOAD = RMSN_LOAD_AUX;
constexpr int AUX_STREAM_STORE = RMSN_STORE_AUX;
constexpr int AUX_SINGLE_STORE = RMSN_SINGLE_STORE_AUX;  // plain and LayerNorm dx, shorter rows
constexpr int AUX_FWD_STORE = RMSN_FWD_STORE_AUX;              // the forwards' y
constexpr int AUX_FWD_SHORT_STORE = RMSN_FWD_SHORT_STORE_AUX;  // y of rows short a thread

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, RSRC_WORD3);
}

template <int DT, int VEC, int AUX>
__device__ __forceinline__ Pack<DT, VEC> buf_load(rsrc_t r, uint32_t off) {
    constexpr int B = Pack<DT, VEC>::BYTES;
    Pack<DT, VEC> p;
    if constexpr (B == 16) {
        p.v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    } else if constexpr (B == 8) {
        p.v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    } else if constexpr (B == 4) {
        p.v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
    } else {
        p.v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
    }
    return p;
}

template <int DT, int VEC, int AUX>
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t off, const Pack<DT, VEC> &p) {
    constexpr int B = Pack<DT, VEC>::BYTES;
    if constexpr (B == 16) {
        __builtin_amdgcn_raw_buffer_store_b128(p.v, r, off, 0, AUX);
    } else if constexpr (B == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(p.v, r, off, 0, AUX);
    } else if constexpr (B == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(p.v, r, off, 0, AUX);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16(p.v, r, off, 0, AUX);
    }
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX_DEFAULT));
}

__device__ __forceinline__ void buf_store_f32(rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, AUX_DEFAULT);
}

// ---------------------------------------------------------------------------
// Row windows: a window is the RPB consecutive rows one block handles in a
// step, one per row group.
// ---------------------------------------------------------------------------
// Byte address of element `elem` of a tensor, as an integer: window bases may
// lie past the end of a tensor when the window holds no row (its descriptor
// range is then empty and nothing is accessed).
__device__ __forceinline__ const void *at(const void *base, int64_t elem, int es) {
    return reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(base) + (uintptr_t)(elem * es));
}

// Buffer descriptor for one window of a row tensor with row stride ld
// elements: rows wb .. wb + nr - 1 exist, and the range ends at the end of the
// last of them, so rows past M, chunks past N and the gap between strided rows
// all fall outside it.
template <int ES>
__device__ __forceinline__ rsrc_t window_rsrc(const void *base, int64_t wb, int64_t ld, uint32_t nr,
                                              uint32_t row_bytes) {
    const uint32_t span = nr == 0 ? 0u : (uint32_t)((int64_t)(nr - 1) * ld * ES) + row_bytes;
    return make_rsrc(at(base, wb * ld, ES), span);
}

// Rows of the window starting at row wb that exist: min(RPB, M - wb), >= 0.
template <int RPB>
__device__ __forceinline__ uint32_t rows_in(int64_t wb, int64_t M) {
    const int64_t r = M - wb;
    return r <= 0 ? 0u : (r >= RPB ? (uint32_t)RPB : (uint32_t)r);
}

template <int DT, int VEC>
__device__ __forceinline__ Pack<DT, VEC> zero_pack() {
    Pack<DT, VEC> p;
    if constexpr (Pack<DT, VEC>::BYTES >= 8) {
#pragma unroll
        for (int w = 0; w < Pack<DT, VEC>::BYTES / 4; ++w) p.v[w] = 0u;
    } else {
        p.v = 0;
    }
    return p;
}

// An empty asm statement that claims to rewrite the packs' registers: values
// derived from them before this point cannot be reused after it, so the
// compiler recomputes them instead of keeping them live.
template <int DT, int VEC>
__device__ __forceinline__ void opaque(Pack<DT, VEC> &a, Pack<DT, VEC> &b) {
    asm volatile("" : "+v"(a.v), "+v"(b.v));
}

// An empty asm statement that reads the pack's registers: every load still
// in flight into them must have arrived before this point.
template <int DT, int VEC>
__device__ __forceinline__ void consume(const Pack<DT, VEC> &a) {
    asm volatile("" : : "v"(a.v));
}

// Ends a window's arithmetic: its packed results exist before this point and
// no memory access moves across it. Without it the compiler hoists the next
// window's loads above the last uses of the current window's registers, and
// the ring slot then needs a register copy at the loop's back edge, which
// must wait for those loads.
template <int DT, int VEC, int K>
__device__ __forceinline__ void settle(const Pack<DT, VEC> (&out)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) asm volatile("" : : "v"(out[k].v) : "memory");
}

// ---------------------------------------------------------------------------
// Cross-lane sums. Every lane of an aligned group of W lanes (W a power of two,
// 16 <= W <= 64) ends with the group's total. Each lane's order of additions
// is fixed, so results repeat bit for bit from call to call; for W < 64 lanes
// of one group may associate the partial sums differently and so differ in
// the last bit. For W = 64 every lane holds the same value.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W == 16 || W == 32 || W == 64, "group width");
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_mov<0x124>(v);  // row_ror:4 inside each 16-lane row
    v += dpp_mov<0x128>(v);  // row_ror:8
    if constexpr (W >= 32) {
        // ds_swizzle, bit mode, xor mask 16 (within 32-lane halves)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    }
    if constexpr (W == 64) {
        // both 32-lane halves now hold their half's total; v_readlane_b32
        // reads each, and every lane adds them in the same order
        v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    }
    return v;
}

}  // namespace rmsn
