// Device-side helpers shared by the normhip kernels (gfx950, wave64).
//
// Storage types: `float` for fp32 and `uint16_t` bit patterns for bf16.  All
// arithmetic happens in fp32 registers; bf16 is widened on load (exact) and
// narrowed on store with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nh {

constexpr int kWave = 64;

// ---- scalar conversions ---------------------------------------------------

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// ---- vector loads/stores of V consecutive elements --------------------------
// p must be aligned to V*sizeof(T) bytes when V > 1.

template <typename T, int V> struct Vec;

template <> struct Vec<float, 1> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[1]) { o[0] = *p; }
    static __device__ __forceinline__ void store(float *p, const float (&v)[1]) { *p = v[0]; }
};
template <> struct Vec<float, 4> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[4])
    {
        float4 v = *reinterpret_cast<const float4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[4])
    {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Vec<float, 8> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[8])
    {
        float4 a = reinterpret_cast<const float4 *>(p)[0];
        float4 b = reinterpret_cast<const float4 *>(p)[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[8])
    {
        reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
};

__device__ __forceinline__ void unpack_bf16x2(uint32_t u, float &lo, float &hi)
{
    lo = __uint_as_float(u << 16);
    hi = __uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)from_f32<uint16_t>(lo) | ((uint32_t)from_f32<uint16_t>(hi) << 16);
}

template <> struct Vec<uint16_t, 1> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[1]) { o[0] = to_f32(*p); }
    static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[1]) { *p = from_f32<uint16_t>(v[0]); }
};
template <> struct Vec<uint16_t, 4> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[4])
    {
        uint2 u = *reinterpret_cast<const uint2 *>(p);
        unpack_bf16x2(u.x, o[0], o[1]);
        unpack_bf16x2(u.y, o[2], o[3]);
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[4])
    {
        *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
};
template <> struct Vec<uint16_t, 8> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[8])
    {
        uint4 u = *reinterpret_cast<const uint4 *>(p);
        unpack_bf16x2(u.x, o[0], o[1]);
        unpack_bf16x2(u.y, o[2], o[3]);
        unpack_bf16x2(u.z, o[4], o[5]);
        unpack_bf16x2(u.w, o[6], o[7]);
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[8])
    {
        *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};

template <typename T, int V>
__device__ __forceinline__ void load_vec(const T *p, float (&o)[V]) { Vec<T, V>::load(p, o); }
template <typename T, int V>
__device__ __forceinline__ void store_vec(T *p, const float (&v)[V]) { Vec<T, V>::store(p, v); }

// ---- nontemporal (streaming) variants ---------------------------------------------
// Loads and stores that carry the nontemporal hint: on MI355X a stream that is
// touched once moves through the caches markedly faster this way (plain
// stores in particular), measured on 33-537 MB streams.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t nt_load(const f32x4_t *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x4_t nt_load(const u32x4_t *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2_t nt_load(const u32x2_t *p) { return __builtin_nontemporal_load(p); }

template <bool NT, typename T, int V> struct VecNT;

template <typename T, int V> struct VecNT<false, T, V> {
    static __device__ __forceinline__ void load(const T *p, float (&o)[V]) { Vec<T, V>::load(p, o); }
    static __device__ __forceinline__ void store(T *p, const float (&v)[V]) { Vec<T, V>::store(p, v); }
};
template <> struct VecNT<true, float, 1> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[1]) { o[0] = __builtin_nontemporal_load(p); }
    static __device__ __forceinline__ void store(float *p, const float (&v)[1]) { __builtin_nontemporal_store(v[0], p); }
};
template <> struct VecNT<true, uint16_t, 1> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[1]) { o[0] = to_f32((uint16_t)__builtin_nontemporal_load(p)); }
    static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[1]) { __builtin_nontemporal_store(from_f32<uint16_t>(v[0]), p); }
};
template <> struct VecNT<true, float, 4> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[4])
    {
        f32x4_t v = nt_load(reinterpret_cast<const f32x4_t *>(p));
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[4])
    {
        f32x4_t t = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t *>(p));
    }
};
template <> struct VecNT<true, float, 8> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[8])
    {
        f32x4_t a = nt_load(reinterpret_cast<const f32x4_t *>(p));
        f32x4_t b = nt_load(reinterpret_cast<const f32x4_t *>(p) + 1);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[8])
    {
        f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t *>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t *>(p) + 1);
    }
};
template <> struct VecNT<true, uint16_t, 4> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[4])
    {
        u32x2_t u = nt_load(reinterpret_cast<const u32x2_t *>(p));
        unpack_bf16x2(u.x, o[0], o[1]);
        unpack_bf16x2(u.y, o[2], o[3]);
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[4])
    {
        u32x2_t t = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t *>(p));
    }
};
template <> struct VecNT<true, uint16_t, 8> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[8])
    {
        u32x4_t u = nt_load(reinterpret_cast<const u32x4_t *>(p));
        unpack_bf16x2(u.x, o[0], o[1]);
        unpack_bf16x2(u.y, o[2], o[3]);
        unpack_bf16x2(u.z, o[4], o[5]);
        unpack_bf16x2(u.w, o[6], o[7]);
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[8])
    {
        u32x4_t t = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
        __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t *>(p));
    }
};

template <bool NT, typename T, int V>
__device__ __forceinline__ void ld(const T *p, float (&o)[V]) { VecNT<NT, T, V>::load(p, o); }
template <bool NT, typename T, int V>
__device__ __forceinline__ void st(T *p, const float (&v)[V]) { VecNT<NT, T, V>::store(p, v); }

// ---- packed storage of V loaded elements -----------------------------------------
// Keeps a loaded vector in its storage form (bf16 stays two-per-register) and
// widens one element at a time, so a row held across a reduction costs
// V*sizeof(T) bytes of registers, not V*4.
template <typename T, int V> struct Raw;

template <typename T, int V> struct BufLoad;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes);

template <int V> struct Raw<float, V> {
    float v[V];
    __device__ __forceinline__ void load(const float *p) { Vec<float, V>::load(p, v); }
    __device__ __forceinline__ void load_nt(const float *p) { VecNT<true, float, V>::load(p, v); }
    // Nontemporal, range-checked load at byte offset `off` of buffer `r`.
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) { BufLoad<float, V>::load(r, off, v); }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
};

// A single bf16 element, kept as its bit pattern until widened.
template <> struct Raw<uint16_t, 1> {
    uint32_t u;
    __device__ __forceinline__ void load(const uint16_t *p) { u = *p; }
    __device__ __forceinline__ void load_nt(const uint16_t *p) { u = (uint16_t)__builtin_nontemporal_load(p); }
    __device__ __forceinline__ float get(int) const { return __uint_as_float(u << 16); }
};

template <int V> struct Raw<uint16_t, V> {
    static_assert(V == 4 || V == 8, "bf16 groups hold 4 or 8 elements");
    uint32_t u[V / 2];
    __device__ __forceinline__ void load(const uint16_t *p)
    {
        if constexpr (V == 8) {
            uint4 t = *reinterpret_cast<const uint4 *>(p);
            u[0] = t.x; u[1] = t.y; u[2] = t.z; u[3] = t.w;
        } else {
            uint2 t = *reinterpret_cast<const uint2 *>(p);
            u[0] = t.x; u[1] = t.y;
        }
    }
    __device__ __forceinline__ void load_nt(const uint16_t *p);
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off);
    __device__ __forceinline__ float get(int e) const
    {
        const uint32_t w = u[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// ---- wave64 reductions ------------------------------------------------------
// Butterfly over xor distances 32..1: every lane ends with the same bits
// (IEEE addition is commutative, so the two partners of each exchange form
// identical sums), and the order is fixed, so results repeat run to run.

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---- DPP wave sums -------------------------------------------------------------
// DPP lane selections inside a row of 16 lanes (gfx9 encodings): quad_perm
// [1,0,3,2] (lane i <-> i^1) and [2,3,0,1] (i <-> i^2), row_half_mirror
// (i <-> 7-i in each half row) and row_mirror (i <-> 15-i).
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// v plus the v of the partner lane that CTRL selects.  The partners pair up,
// so both sides add the same two values.
template <int CTRL>
__device__ __forceinline__ float dpp_pair_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// The fp64 form moves the two 32-bit halves with one DPP selection each.
template <int CTRL>
__device__ __forceinline__ double dpp_pair_add(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes of a wave, the same in every lane: DPP steps give
// every lane its 16-lane row's sum, then the four row sums (lanes 0, 16, 32,
// 48) are added pairwise, (r0 + r1) + (r2 + r3).  All lanes must be active.
// A DPP step is a register operand of the add, so the four in-row steps take
// no LDS round trip (the __shfl_xor butterfly above takes six).
__device__ __forceinline__ float wave_total(float v)
{
    v = dpp_pair_add<kDppRowMirror>(v);
    v = dpp_pair_add<kDppRowHalfMirror>(v);
    v = dpp_pair_add<kDppQuadXor2>(v);
    v = dpp_pair_add<kDppQuadXor1>(v);
    const int u = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(u, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(u, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(u, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(u, 48));
    return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ double wave_total(double v)
{
    v = dpp_pair_add<kDppRowMirror>(v);
    v = dpp_pair_add<kDppRowHalfMirror>(v);
    v = dpp_pair_add<kDppQuadXor2>(v);
    v = dpp_pair_add<kDppQuadXor1>(v);
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    auto row = [&](int lane) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
        return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    };
    return (row(0) + row(16)) + (row(32) + row(48));
}

// ---- workgroup barrier for LDS traffic only ---------------------------------------
// __syncthreads() orders every address space, so it also waits for all of the
// wave's outstanding global loads (s_waitcnt vmcnt(0)) -- including loads
// issued ahead for the next row.  Where only LDS data is exchanged, fence LDS
// alone: the barrier then leaves prefetched global loads in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- fast unsigned division by a run-time invariant --------------------------
// Granlund & Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994): with s = ceil(log2 d) and
// m = floor(2^32 * (2^s - d) / d) + 1, n / d = (mulhi(n, m) + n) >> s.
// The sum mulhi(n, m) + n stays below 2^32 for n < 2^31, the only range used.
struct FastDiv {
    uint32_t d;
    uint32_t m;
    uint32_t s;

    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const
    {
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t hi = __umulhi(n, m);
#else
        uint32_t hi = (uint32_t)(((uint64_t)n * (uint64_t)m) >> 32);
#endif
        return (hi + n) >> s;
    }
};

// ---- buffer loads: range-checked without branches ----------------------------------
// A raw buffer resource covers [base, base + bytes); a load at an offset past
// that range returns zeros and touches no memory.  Loads guarded this way
// stay in straight-line code, which lets the compiler wait for exactly the
// older loads instead of draining all of them at every control-flow merge.
// The descriptor's last word (0x00020000: 32-bit data format, raw access) is
// the gfx9-family value; aux = 2 sets the nontemporal bit.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}

template <typename T, int V> struct BufLoad;
template <> struct BufLoad<float, 4> {
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off, float (&o)[4])
    {
        u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufferNT);
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
};
template <> struct BufLoad<float, 8> {
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off, float (&o)[8])
    {
        u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufferNT);
        u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kBufferNT);
        o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
        o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
        o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y);
        o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
    }
};

template <int V>
__device__ __forceinline__ void Raw<uint16_t, V>::load_nt(const uint16_t *p)
{
    if constexpr (V == 8) {
        u32x4_t t = nt_load(reinterpret_cast<const u32x4_t *>(p));
        u[0] = t.x; u[1] = t.y; u[2] = t.z; u[3] = t.w;
    } else {
        u32x2_t t = nt_load(reinterpret_cast<const u32x2_t *>(p));
        u[0] = t.x; u[1] = t.y;
    }
}

template <int V>
__device__ __forceinline__ void Raw<uint16_t, V>::load_buf(__amdgpu_buffer_rsrc_t r, int off)
{
    if constexpr (V == 8) {
        u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufferNT);
        u[0] = t.x; u[1] = t.y; u[2] = t.z; u[3] = t.w;
    } else {
        u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kBufferNT);
        u[0] = t.x; u[1] = t.y;
    }
}

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    f.s = 0;
    while ((1ull << f.s) < (uint64_t)d) ++f.s;
    f.m = (uint32_t)((((1ull << 32) * ((1ull << f.s) - (uint64_t)d)) / (uint64_t)d) + 1ull);
    return f;
}

} // namespace nh
