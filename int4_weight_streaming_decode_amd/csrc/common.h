// Device helpers shared by the decode kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32;
typedef uint64_t u64;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

#define I4D_DEVINL __device__ __forceinline__

// Thread index as an opaque value: the persistent kernel runs every phase of
// every layer in one loop, and without this the compiler hoists each phase's
// lane arithmetic out of the layer loop and keeps all of it live at once.
I4D_DEVINL int i4d_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Loads and stores through global-address-space pointers.  The persistent
// kernel reads its matrix and cache pointers from a table in device memory,
// and for such pointers the compiler would emit flat instructions, which also
// count against the LDS wait counter: every LDS wait would then wait for the
// weight stream as well.
#define I4D_GLOBAL __attribute__((address_space(1)))
#define I4D_CONST __attribute__((address_space(4)))
template <class T> I4D_DEVINL T ld_g(const T* p) { return *(const I4D_GLOBAL T*)p; }
template <class T> I4D_DEVINL void st_g(T* p, T v) { *(I4D_GLOBAL T*)p = v; }
template <class T> I4D_DEVINL T ld_g_nt(const T* p) { return __builtin_nontemporal_load((const I4D_GLOBAL T*)p); }

// ---------------------------------------------------------------- bf16
I4D_DEVINL float bf16_to_f32(uint16_t b) { return __uint_as_float((u32)b << 16); }

// round-to-nearest-even to bf16 (finite inputs)
I4D_DEVINL uint16_t f32_to_bf16(float f) {
    u32 u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- cross-lane
// Sum over the 16 lanes of a DPP row; every lane of the row gets the total
// (rotations within the row; the same fixed schedule on every call).
I4D_DEVINL float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
    return v;
}

I4D_DEVINL float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
I4D_DEVINL float shfl_f(float v, int lane) { return __shfl(v, lane, 64); }

// ---------------------------------------------------------------- ordered argmax keys
// Larger float -> larger unsigned key; lower index wins ties via the inverted
// index in the low word, so one unsigned max gives (max logit, lowest id).
I4D_DEVINL u32 float_order_key(float f) {
    u32 u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
I4D_DEVINL float float_from_order_key(u32 k) {
    u32 u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}
I4D_DEVINL u64 argmax_key(float logit, u32 idx) { return ((u64)float_order_key(logit) << 32) | (u64)(0xFFFFFFFFu - idx); }

// ---------------------------------------------------------------- temperature sampling
// First output word of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC'11): ten rounds, each multiplying
// words 0 and 2 by the round multipliers and mixing the high halves with words
// 1 and 3 and the round key; the key advances by the Weyl increments between
// rounds.
I4D_DEVINL u32 philox4x32_10_x0(u32 c0, u32 c1, u32 c2, u32 c3, u32 k0, u32 k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const u32 lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const u32 lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        c0 = hi1 ^ c1 ^ k0; c1 = lo1;
        c2 = hi0 ^ c3 ^ k1; c3 = lo0;
    }
    return c0;
}

// The score the LM head's argmax compares.  Greedy (inv_t == 0): the logit.
// Sampling at temperature T = 1 / inv_t (Gumbel-max): logit / T + g with
// g = -log(-log(u)), u = (floor(x / 512) + 1/2) / 2^23 (exact in fp32, strictly
// inside (0, 1)), x = Philox4x32-10 word 0 at counter (row, sequence, ctr[b],
// 0) and key (k0, k1).  The argmax of these scores is a draw from
// softmax(logits / T), so the running argmax serves sampling unchanged.
struct Sampler {
    float inv_t;             // 0: greedy
    u32 k0, k1;              // seed, low and high words
    const int* ctr;          // [B] per-sequence counter word (device memory)
    I4D_DEVINL float score(float logit, int b, u32 row) const {
        if (inv_t == 0.f) return logit;
        const u32 x = philox4x32_10_x0(row, (u32)b, (u32)ctr[b], 0u, k0, k1);
        const float u = ((float)(x >> 9) + 0.5f) * 1.1920928955078125e-7f;     // 2^-23
        return logit * inv_t - logf(-logf(u));
    }
};

// ---------------------------------------------------------------- device-coherent accesses
// Values one workgroup writes and another reads within the same kernel (the
// persistent decode kernel passes activations, q, attention partials and the
// appended K/V between phases) use device-scope accesses: the store writes
// through to memory and the load does not use a possibly stale line of its
// own XCD's L2.  A writer makes its stores visible by waiting for their
// completion (wait_stores) before it raises its barrier flag; no L2 writeback
// fence is needed because none of the exchanged data sits dirty in an L2.
template <class T> I4D_DEVINL void st_dev_t(T* p, T v) { __hip_atomic_store((I4D_GLOBAL T*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <class T> I4D_DEVINL T ld_dev_t(const T* p) { return __hip_atomic_load((I4D_GLOBAL T*)const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
I4D_DEVINL void st_dev(float* p, float v) { st_dev_t(p, v); }
I4D_DEVINL void st_dev(int* p, int v) { st_dev_t(p, v); }
I4D_DEVINL void st_dev(uint16_t* p, uint16_t v) { st_dev_t(p, v); }
I4D_DEVINL void st_dev(u64* p, u64 v) { st_dev_t(p, v); }
// An output store: write-through (st_dev) when workgroups of the same launch
// read it, a plain global store when only a later launch does (the kernel
// boundary makes it visible).
template <bool WT, class T> I4D_DEVINL void st_out(T* p, T v) {
    if constexpr (WT) st_dev_t(p, v);
    else *(I4D_GLOBAL T*)p = v;
}
I4D_DEVINL float ld_dev(const float* p) { return ld_dev_t(p); }
I4D_DEVINL int ld_dev(const int* p) { return ld_dev_t(p); }
I4D_DEVINL u64 ld_dev(const u64* p) { return ld_dev_t(p); }
I4D_DEVINL f4 ld_dev4(const float* p) { return f4{ld_dev(p), ld_dev(p + 1), ld_dev(p + 2), ld_dev(p + 3)}; }
// wait until every vector-memory access of this thread (stores included) has completed
I4D_DEVINL void wait_stores() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt untouched
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- status word
I4D_DEVINL void raise_status(int* status, int bit) { atomicOr(status, bit); }
