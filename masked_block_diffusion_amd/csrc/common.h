// Device-side building blocks shared by the gfx950 kernels: storage types,
// bf16 / OCP E4M3FN conversions written from the formats' definitions, MFMA
// fragment types, and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlm {

typedef uint16_t bf16_t;   // bfloat16 bits
typedef uint8_t fp8_t;     // OCP E4M3FN bits

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest bfloat16, ties to even; overflow -> inf; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// E4M3FN value of a code: sign, 4-bit exponent (bias 7), 3-bit mantissa,
// exponent field 0 = subnormal (m/8 * 2^-6), S.1111.111 = NaN, no infinity.
__device__ __forceinline__ float e4m3_to_f32(fp8_t c) {
    const uint32_t s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    float v;
    if (e == 0xF && m == 7) v = __uint_as_float(0x7fc00000u);
    else if (e == 0) v = (float)m * 0.001953125f;               // m * 2^-9
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1+m/8) * 2^(e-7)
    return s ? -v : v;
}

// Nearest E4M3FN code to a finite fp32 value, ties to even, saturating to
// +-448.  Works on the exact binary value: the 4 kept significand bits are
// found from the fp32 exponent, the rest decide the rounding.
__device__ __forceinline__ fp8_t f32_to_e4m3(float f) {
    uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    u &= 0x7fffffffu;
    if (u >= 0x43e00000u) return (fp8_t)(sign | 0x7Eu);          // |f| >= 448 -> 448
    const int e = (int)(u >> 23) - 127;                           // unbiased exponent
    uint32_t code;
    if (e < -6) {
        // subnormal range: value = q * 2^-9, q = rint(|f| * 2^9) in [0, 8]
        // (|f| < 2^-6; fp32 multiply by a power of two is exact here)
        float q = rintf(__uint_as_float(u) * 512.0f);
        code = (uint32_t)q;                                        // 8 -> 0x08 = 2^-6
    } else {
        // normal: keep 3 mantissa bits, round the other 20 to nearest even
        uint32_t mant = u & 0x7fffffu;
        uint32_t keep = mant >> 20, rest = mant & 0xfffffu;
        uint32_t ex = (uint32_t)(e + 7);
        if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) {
            keep += 1;
            if (keep == 8) { keep = 0; ex += 1; }
        }
        code = (ex << 3) | keep;
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return (fp8_t)(sign | code);
}

// z * sigmoid(z) with the hardware exp2 and reciprocal (each within ~1 ulp);
// z -> -inf gives -0, z -> +inf gives z.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ------------------------------------------------------------ reductions --

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// ---------------------------------------------------------- MFMA traits --
// Per element type: K covered by one step of the 16x16 tile, bytes one lane
// reads per operand and step, the register operand those bytes become, and
// the multiply-accumulate.  bf16 / f32 (one MFMA 16x16xK): lane l supplies row
// (l % 16) of A / column (l % 16) of B, K elements [(l/16) K/4, (l/16) K/4 +
// K/4); the 4 fp32 results of lane l are D[4 (l/16) + i][l % 16], i = 0..3.

template <typename T> struct Mfma;

template <> struct Mfma<float> {
    static constexpr int KSTEP = 4;            // elements per step
    static constexpr int LANE_BYTES = 4;
    typedef float frag;
    typedef float raw;                         // what a lane reads from LDS
    __device__ __forceinline__ static raw load(const uint8_t* p) { return *(const raw*)p; }
    __device__ __forceinline__ static frag widen(raw r) { return r; }
    __device__ __forceinline__ static f32x4 mac(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<bf16_t> {
    static constexpr int KSTEP = 32;
    static constexpr int LANE_BYTES = 16;
    typedef bf16x8 frag;
    typedef bf16x8 raw;
    __device__ __forceinline__ static raw load(const uint8_t* p) { return *(const raw*)p; }
    __device__ __forceinline__ static frag widen(raw r) { return r; }
    __device__ __forceinline__ static f32x4 mac(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// E4M3 operands are widened in registers to bf16 (exact: 4 exponent and 3
// mantissa bits fit bf16's 8 and 7, subnormals included) and multiplied on
// the bf16 MFMA, whose fp32 accumulation meets the fp32 rounding bound; the
// fp8 MFMA's own 32-term sums measured about 2^-15 of sum|ab| off on this
// chip, independent of K.  The bytes in HBM and LDS stay one per element.
// A step covers K = 64: lane l reads codes k = 16 (l/16) .. 16 (l/16) + 15 of
// the step and splits them into two bf16 fragments (the low and high 8);
// A and B use the same assignment, so the two MFMAs add up all 64 products.
__device__ __forceinline__ bf16x8 widen_e4m3x8(uint32_t w0, uint32_t w1) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

template <> struct Mfma<fp8_t> {
    static constexpr int KSTEP = 64;
    static constexpr int LANE_BYTES = 16;
    struct frag { bf16x8 lo, hi; };
    typedef u32x4 raw;                         // 16 codes
    __device__ __forceinline__ static raw load(const uint8_t* p) { return *(const raw*)p; }
    __device__ __forceinline__ static frag widen(raw w) {
        return frag{widen_e4m3x8(w.x, w.y), widen_e4m3x8(w.z, w.w)};
    }
    __device__ __forceinline__ static f32x4 mac(const frag& a, const frag& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.lo, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    }
};

// ------------------------------------------------- LDS-DMA pipelines --

typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt on vector-memory operations only: vmcnt <= N (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Wait until at most p stages (of LPW loads each) are still outstanding.
template <int LPW, int P>
__device__ __forceinline__ void wait_stages(int p) {
    if constexpr (P <= 0) {
        wait_vm<0>();
    } else {
        if (p >= P) wait_vm<P * LPW>();
        else wait_stages<LPW, P - 1>(p);
    }
}

// Workgroup barrier for the LDS ring.  __syncthreads() would add a release
// fence that drains every outstanding LDS-DMA load (all stages in flight);
// here each wave has already waited for the stage it needs, so
// the barrier only has to order LDS reads: lgkmcnt(0), s_barrier, and a
// compiler memory clobber so no LDS access moves across it.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("s_barrier" ::: "memory");
}

// Error word bits (mirrors dlm.h).
constexpr int DEVERR_TOKEN_RANGE = 1;
constexpr int DEVERR_MASK_APPEND = 2;

}  // namespace dlm
