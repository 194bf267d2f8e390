// Device helpers shared by the gfx950 kernels of the sparse-FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte global load (8 fp16 values).
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte streaming load: data read once, marked non-temporal so it does not
// displace reused lines (x, h, partial sums) from the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f16x2 as_h2(unsigned int v) { return __builtin_bit_cast(f16x2, v); }

// A buffer resource over `bytes` bytes at base (raw: stride 0, 32-bit data
// format).  Loads through it take one per-lane offset register and a scalar
// offset, and a 16-byte load at or past `bytes` returns zeros instead of
// touching memory, so a row's tail needs no per-lane branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset voff + soff (soff wave-uniform), non-temporal.
__device__ __forceinline__ u32x4 buf_ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}

// acc + sum_k w[k] * x[k] over 8 fp16 pairs, fp16 products accumulated in fp32
// (v_dot2_f32_f16: the products of two fp16 values are exact in fp32).
__device__ __forceinline__ float dot8_h(u32x4 w, u32x4 x, float acc) {
    acc = __builtin_amdgcn_fdot2(as_h2(w.x), as_h2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w.y), as_h2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w.z), as_h2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w.w), as_h2(x.w), acc, false);
    return acc;
}

// acc + sum_k w[k] * h[k] with fp16 weights and fp32 activations.
__device__ __forceinline__ float dot8_hf(u32x4 w, const float* h, float acc) {
    f16x2 a = as_h2(w.x), b = as_h2(w.y), c = as_h2(w.z), d = as_h2(w.w);
    acc = fmaf((float)a.x, h[0], acc);
    acc = fmaf((float)a.y, h[1], acc);
    acc = fmaf((float)b.x, h[2], acc);
    acc = fmaf((float)b.y, h[3], acc);
    acc = fmaf((float)c.x, h[4], acc);
    acc = fmaf((float)c.y, h[5], acc);
    acc = fmaf((float)d.x, h[6], acc);
    acc = fmaf((float)d.y, h[7], acc);
    return acc;
}

// A neuron's activation from its up sum u and gate sum g (biases included),
// by FFN kind: 0 ReLU max(u, 0); 1 ReGLU max(g, 0) * u; 2 SwiGLU SiLU(g) * u
// with SiLU(g) = g / (1 + e^-g).
template <int KIND>
__device__ __forceinline__ float ffn_act(float u, float g) {
    if (KIND == 0) return fmaxf(u, 0.f);
    if (KIND == 1) return fmaxf(g, 0.f) * u;
    return g / (1.f + expf(-g)) * u;
}

// sum_j (code_j - 8) * x_j over the 8 weights of one 32-bit code word and 8
// fp16 x.  The codes become fp16 pairs without conversions: a byte permute
// puts codes 2j and 2j + 1 in the low bytes of the two halves, or-ing in
// 0x6400 makes them 1024 + code (exact in fp16), and one packed subtraction
// of 1032 leaves code - 8; the pairs go through the fp16 dot product with
// fp32 accumulation (products of fp16 values are exact in fp32).
__device__ __forceinline__ float dot8_q4(uint32_t codes, u32x4 x, float acc) {
    const uint32_t lo = codes & 0x0F0F0F0Fu;          // codes of weights 0, 2, 4, 6 (byte j: weight 2j)
    const uint32_t hi = (codes >> 4) & 0x0F0F0F0Fu;   // codes of weights 1, 3, 5, 7
    const f16x2 off = {(f16)1032.0f, (f16)1032.0f};
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // result bytes: lo byte j, 0, hi byte j, 0 (perm: bytes 0-3 of the second
        // operand are 0-3, of the first 4-7; 0x0C selects a zero byte)
        const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + j) << 16) | (uint32_t)j;
        const uint32_t p = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
        acc = __builtin_amdgcn_fdot2(as_h2(p) - off, as_h2(xs[j]), acc, false);
    }
    return acc;
}

// acc[e] += f * (code_e - 8) for the 8 4-bit codes of one word (INT4 rows;
// f is the activation times the group's scale).
__device__ __forceinline__ void axpy8_q4(float* acc, float f, uint32_t codes) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(f, (float)((int)((codes >> (4 * e)) & 0xFu) - 8), acc[e]);
}

// acc[k] += s * w[k] for 8 fp16 weights.
__device__ __forceinline__ void axpy8(float* acc, float s, u32x4 w) {
    f16x2 a = as_h2(w.x), b = as_h2(w.y), c = as_h2(w.z), d = as_h2(w.w);
    acc[0] = fmaf(s, (float)a.x, acc[0]);
    acc[1] = fmaf(s, (float)a.y, acc[1]);
    acc[2] = fmaf(s, (float)b.x, acc[2]);
    acc[3] = fmaf(s, (float)b.y, acc[3]);
    acc[4] = fmaf(s, (float)c.x, acc[4]);
    acc[5] = fmaf(s, (float)c.y, acc[5]);
    acc[6] = fmaf(s, (float)d.x, acc[6]);
    acc[7] = fmaf(s, (float)d.y, acc[7]);
}

// v plus the v of the lane that the DPP control CTRL pairs with this lane
// (a partner inside the same 16-lane row, so always in range).  A VALU
// operand modifier: no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// v[lane] + v[lane ^ 16] (S = 16) or v[lane] + v[lane ^ 32] (S = 32): the
// gfx950 permlane swaps exchange the odd 16-lane rows of one operand with the
// even rows of the other (S = 16), or the upper 32 lanes with the lower 32
// (S = 32).  With both operands v, each lane ends up holding its own value in
// one result and its partner's in the other.
template <int S>
__device__ __forceinline__ float add_swap(float v) {
    const uint32_t u = __float_as_uint(v);
    if constexpr (S == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of a
// group ends with the group sum.  Inside a 16-lane row the partners come from
// DPP: lane ^ 1, lane ^ 2 (quad permutes), then the mirror inside each 8-lane
// half (i <-> 7 - i) and inside the row (i <-> 15 - i).  After each step a
// lane holds the sum of a block twice the size, because each mirror pairs
// every lane with one in the other half of that block.  Rows are then joined
// across 16 and 32 lanes by the permlane swaps.  All VALU, no LDS round trip.
// Called with every lane of the wave active.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: a power of two up to the wave");
    if constexpr (W >= 2) v = add_dpp<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    if constexpr (W >= 4) v = add_dpp<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    if constexpr (W >= 8) v = add_dpp<0x141>(v);   // row_half_mirror
    if constexpr (W >= 16) v = add_dpp<0x140>(v);  // row_mirror
    if constexpr (W >= 32) v = add_swap<16>(v);
    if constexpr (W >= 64) v = add_swap<32>(v);
    return v;
}

template <int W>
__device__ __forceinline__ uint32_t group_sum_u32(uint32_t v) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ uint32_t rank_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// A list length clamped to [0, ffn], a neuron id to [0, ffn): a broken list
// can never make a kernel read outside the weights.
__device__ __forceinline__ int clamp_count(int c, int ffn) { return c < 0 ? 0 : (c > ffn ? ffn : c); }
__device__ __forceinline__ int clamp_row(int i, int ffn) { return i < 0 ? 0 : (i >= ffn ? ffn - 1 : i); }

// Device-coherent relaxed accesses for cross-workgroup flags.
__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_acq_rel(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
// Load that observes the device-coherent value (no stale per-XCD cache line).
__device__ __forceinline__ float ld_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Returns v as a plain register value: the compiler waits for the load that
// produced it here, once, rather than before each later use it has sunk into
// a branch (there it cannot count the loads and waits for every outstanding
// memory operation, the stores issued since included).
template <class T>
__device__ __forceinline__ T settle(T v) {
    asm volatile("" : "+v"(v));
    return v;
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_own_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// at their maximum so they are not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// Direct-to-LDS load of 16 bytes per lane (global_load_lds_dwordx4: lane l's
// bytes land at lds_addr + 16 l; lds_addr is wave-uniform, it goes to M0),
// issued as inline assembly.  Were the compiler to see it, it would make every
// LDS read wait for all outstanding vector-memory loads (it cannot tell which
// LDS bytes the load writes); the caller orders the load and the reads with
// its own waits and barriers instead.  (A load the compiler does not count can
// only make its own waits stricter.)  dma16_coherent reads the device-coherent
// value, as the relaxed agent-scope atomic loads do.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds_addr), "v"(gptr) : "memory", "m0");
}
// dma16_stream marks the line non-temporal: a weight byte is read once, so
// the line is the first to go from L2, and the activations that every
// workgroup re-reads stay resident there.
__device__ __forceinline__ void dma16_stream(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" : : "s"(lds_addr), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ void dma16_coherent(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off sc1" : : "s"(lds_addr), "v"(gptr)
                 : "memory", "m0");
}
// The 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)(const char*)p;
}

}  // namespace pi
