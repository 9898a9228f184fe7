// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace q4k {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Bytes of one Q4_0 / Q8_0 block of 32 elements.
constexpr int kQ4Bytes = 18;
constexpr int kQ8Bytes = 34;

// 32-bit load from an address that is only 2-byte aligned. The HSA ABI runs
// gfx9 wavefronts in unaligned-access mode, so this is one global_load_dword.
__device__ __forceinline__ uint32_t load_u32_unaligned(const uint8_t *p)
{
    uint32_t v;
    __builtin_memcpy(&v, p, 4);
    return v;
}

// 16-bit load from a 2-byte aligned address.
__device__ __forceinline__ uint32_t load_u16(const uint8_t *p)
{
    return *reinterpret_cast<const uint16_t *>(p);
}

// Widen a binary16 bit pattern to f32 (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(f16, (uint16_t)bits);
}

// f32 -> binary16 bit pattern, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float v)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (f16)v);
}

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u)
{
    static_assert(sizeof(T) == sizeof(U), "size mismatch");
    return __builtin_bit_cast(T, u);
}

// Launch a kernel and return the runtime's verdict on this launch alone. Each
// argument is first converted to the kernel's own parameter type.
template <typename Kernel, typename Tuple, size_t... I>
inline hipError_t launch_tuple(Kernel kernel, dim3 grid, dim3 block, size_t lds_bytes,
                               hipStream_t stream, Tuple &vals, std::index_sequence<I...>)
{
    void *argv[] = {reinterpret_cast<void *>(&std::get<I>(vals))...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds_bytes,
                           stream);
}

template <typename... Params, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds_bytes,
                                hipStream_t stream, Args &&...args)
{
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    std::tuple<std::decay_t<Params>...> vals(std::forward<Args>(args)...);
    return launch_tuple(kernel, grid, block, lds_bytes, stream, vals,
                        std::index_sequence_for<Params...>{});
}

}  // namespace q4k
