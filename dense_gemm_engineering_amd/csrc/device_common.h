// Device-side helpers shared by the gfx950 kernels: storage types, vector
// bit casts, output rounding and the fused epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dge {

// Input element types (match gemm_in_t) and output types (match gemm_out_t).
enum : int { IN_F16 = 0, IN_BF16 = 1, IN_F32 = 2 };
enum : int { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2 };
enum : int { EPI_NONE = 0, EPI_BIAS = 1, EPI_BIAS_GELU = 2 };
// block-quantised weight formats (numbered as gemm_qtype_t); KQ_Q4_0_256 is
// internal: q4_0 rows whose length is a multiple of 256, walked as groups of
// eight 18-byte blocks (144 bytes per 256 weights)
enum : int { KQ_Q4_0 = 0, KQ_Q4_K = 1, KQ_Q6_K = 2, KQ_Q6_K_224 = 3, KQ_Q4_0_256 = 4 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct InType;
template <> struct InType<IN_F16> {
    static constexpr int BYTES = 2;
    __device__ static inline float to_f32(uint32_t bits) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    }
};
template <> struct InType<IN_BF16> {
    static constexpr int BYTES = 2;
    __device__ static inline float to_f32(uint32_t bits) {
        return __builtin_bit_cast(float, bits << 16);  // bf16 is the top half of fp32
    }
};
template <> struct InType<IN_F32> {
    static constexpr int BYTES = 4;
    __device__ static inline float to_f32(uint32_t bits) { return __builtin_bit_cast(float, bits); }
};

// Load one element of an input array as raw bits (zero-extended).
template <int DT>
__device__ inline uint32_t load_elem_bits(const void* base, int64_t idx) {
    if constexpr (InType<DT>::BYTES == 2)
        return ((const uint16_t*)base)[idx];
    else
        return ((const uint32_t*)base)[idx];
}

template <int DT>
__device__ inline float load_elem(const void* base, int64_t idx) {
    return InType<DT>::to_f32(load_elem_bits<DT>(base, idx));
}

// Output element type: size and one round-to-nearest-even conversion.
template <int OT> struct OutType;
template <> struct OutType<OUT_F32> {
    static constexpr int BYTES = 4;
    typedef float T;
    __device__ static inline float from_f32(float x) { return x; }
    __device__ static inline float to_f32(float x) { return x; }
};
template <> struct OutType<OUT_F16> {
    static constexpr int BYTES = 2;
    typedef _Float16 T;
    __device__ static inline _Float16 from_f32(float x) { return (_Float16)x; }
    __device__ static inline float to_f32(_Float16 x) { return (float)x; }
    // two values rounded to nearest-even and packed, a in the low half: one
    // v_cvt_pk_f16_f32
    __device__ static inline uint32_t pack2(float a, float b) {
        typedef _Float16 v2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, (v2){(_Float16)a, (_Float16)b});
    }
};
template <> struct OutType<OUT_BF16> {
    static constexpr int BYTES = 2;
    typedef __bf16 T;
    __device__ static inline __bf16 from_f32(float x) { return (__bf16)x; }
    __device__ static inline float to_f32(__bf16 x) { return (float)x; }
    __device__ static inline uint32_t pack2(float a, float b) {
        typedef __bf16 v2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, (v2){(__bf16)a, (__bf16)b});
    }
};

// tanh form of GELU: 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))), in fp32.
// With 0.5 (1 + tanh(u)) = 1 / (1 + e^{-2u}) this is t / (1 + 2^x),
// x = -2 log2(e) sqrt(2/pi) (t + 0.044715 t^3) = t (C1 + C2 t^2): three
// multiply-adds, the hardware exp2 and reciprocal (about 1 ulp each, ample
// for a value rounded to 16 bits) and a final product.  It saturates
// correctly: 2^x -> inf gives t * 0 = -0 for large negative t, 2^x -> 0
// gives t.
__device__ inline float gelu_tanh(float t) {
    constexpr float C1 = -2.3022082f;   // -2 log2(e) sqrt(2/pi)
    constexpr float C2 = -0.10294324f;  // C1 * 0.044715
    const float x = t * __builtin_fmaf(C2, t * t, C1);
    return t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

// Epilogue parameters, passed by value to every kernel that ends in C.
struct Epilogue {
    float alpha, beta;
    int epi;           // EPI_*
    const void* bias;  // N values of the input type, or null
};

// The fused epilogue on one accumulator value: alpha*acc + beta*old, + bias,
// then GELU.  `old` is only meaningful when beta != 0.
// epilogue_value takes the bias value already loaded (read only when epi
// adds one); both give the same bits for the same inputs.
__device__ inline float epilogue_value(const Epilogue& e, float acc, float old, float bias) {
    float t = e.alpha * acc;
    if (e.beta != 0.0f) t += e.beta * old;
    if (e.epi != EPI_NONE) t += bias;
    if (e.epi == EPI_BIAS_GELU) t = gelu_tanh(t);
    return t;
}
template <int DT>
__device__ inline float apply_epilogue(const Epilogue& e, float acc, float old, int col) {
    float t = e.alpha * acc;
    if (e.beta != 0.0f) t += e.beta * old;
    if (e.epi != EPI_NONE) t += load_elem<DT>(e.bias, col);
    if (e.epi == EPI_BIAS_GELU) t = gelu_tanh(t);
    return t;
}

// Map a linear workgroup id to a tile so that the workgroups dispatched to
// one XCD (ids congruent mod 8 go to the same XCD) cover a compact block of
// output tiles, ordered in groups of `group_m` tile rows: tiles that share
// an A row panel or a B column panel then meet in the same 4 MB L2.
__device__ inline int remap_xcd(int pid, int nwg) {
    constexpr int NXCD = 8;
    int per = (nwg + NXCD - 1) / NXCD;
    int tall = nwg % NXCD;
    if (tall == 0) tall = NXCD;
    int xcd = pid % NXCD, local = pid / NXCD;
    if (xcd < tall) return xcd * per + local;
    return tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ inline void grouped_tile(int lin, int tiles_m, int tiles_n, int group_m, int& tm,
                                    int& tn) {
    int in_group = group_m * tiles_n;
    int g = lin / in_group;
    int first_m = g * group_m;
    int gsize = tiles_m - first_m;
    if (gsize > group_m) gsize = group_m;
    int r = lin % in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

}  // namespace dge
