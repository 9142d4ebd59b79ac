// Device-side helpers shared by the matrix-core kernels: buffer resources
// with hardware range checking, direct global->LDS loads, wait counters,
// and the workgroup -> output-tile mapping.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>
#include <cstdint>

namespace mmrelu {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MMRELU_LDS __attribute__((address_space(3)))

// Data-format word of a gfx9 buffer resource (32-bit untyped elements).
constexpr uint32_t kBufferFormat = 0x00020000u;
// Per-lane offset that is always past a resource's range: loads return 0
// (direct-to-LDS loads write 0) and stores are dropped.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Largest byte range given to one resource; every valid per-lane offset is
// below it, so kOutOfRange is never inside a range.
constexpr int64_t kMaxRange = 0x7FFFFF00;

// Buffer resource over [base, base + bytes) as four scalar words (base
// address, stride 0, byte range, data format); bytes is clamped to kMaxRange.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ inline rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRange ? kMaxRange : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    rsrc_t r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(a));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((a >> 32) & 0xFFFF));
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(n));
    r[3] = static_cast<int32_t>(kBufferFormat);
    return r;
}

// LDS byte address of a __shared__ object (for M0).
template <typename T>
__device__ inline uint32_t lds_address(const T *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const MMRELU_LDS T *)p));
}

// Direct global -> LDS copy: lane l writes 16 (or 4) bytes at LDS byte
// address lds + l * 16 (or 4); `lds` must be wave-uniform, `soffset` is a
// uniform byte offset added to every lane's voffset. A lane whose offset is
// out of the resource's range writes zeros.
//
// Issued as inline assembly on purpose: the compiler cannot tell which LDS
// bytes such a copy writes, and for the builtin it waits for every copy in
// flight before any later LDS read, which would serialise the prefetch of
// slab k+1 with the multiply of slab k. Completion is awaited explicitly
// (wait_vmcnt + barrier) before a stage is read; the "memory" clobber keeps
// the compiler from moving LDS accesses across the copy.
// M0 is declared clobbered; the kernels make no other use of M0 (no LDS
// builtins that take it, no dynamic register indexing). An LDS copy must not
// directly follow the SALU write of M0 (one wait state, as the compiler
// itself inserts for the builtin form), hence the s_nop.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int Bytes>
__device__ inline void load_to_lds(rsrc_t r, uint32_t lds, uint32_t voffset, uint32_t soffset = 0)
{
    static_assert(Bytes == 4 || Bytes == 16, "4- or 16-byte lanes");
    // Both scalar operands are wave-uniform; keep them in SGPRs even when
    // they are compile-time constants (a buffer soffset literal outside the
    // inline-constant range is not encodable).
    lds = __builtin_amdgcn_readfirstlane(lds);
    soffset = __builtin_amdgcn_readfirstlane(soffset);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    asm("" : "+s"(lds), "+s"(soffset));
    if constexpr (Bytes == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                     :: "v"(voffset), "s"(lds), "s"(r), "s"(soffset) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, %3 offen lds"
                     :: "v"(voffset), "s"(lds), "s"(r), "s"(soffset) : "memory", "m0");
}
// The same copy with no scalar offset (the inline constant 0 in its place,
// which saves the scalar register move per copy). The LDS address needs no
// pinning to a register here: it is only moved into M0, which takes a
// literal as well (an empty asm that pinned it made the compiler put a wait
// state before every copy).
template <int Bytes>
__device__ inline void load_to_lds_z(rsrc_t r, uint32_t lds, uint32_t voffset)
{
    static_assert(Bytes == 4 || Bytes == 16, "4- or 16-byte lanes");
    lds = __builtin_amdgcn_readfirstlane(lds);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    if constexpr (Bytes == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                     :: "v"(voffset), "s"(lds), "s"(r) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
                     :: "v"(voffset), "s"(lds), "s"(r) : "memory", "m0");
}
#pragma clang diagnostic pop

// Store resource over [base, base + bytes) for the masked epilogue stores:
// lanes with an out-of-range offset store nothing.
__device__ inline __amdgpu_buffer_rsrc_t make_store_rsrc(void *base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRange ? kMaxRange : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(n), kBufferFormat);
}
// Fused epilogue, applied to each fp32 accumulator before the one store:
// add the output column's bias (zero without a bias), then the activation.
// Activation codes are those of mmrelu.h: 0 ReLU, 1 GeLU in its tanh form,
// 2 none. GeLU's tanh form is 0.5 x (1 + tanh(u)), u = 0.79788456 (x +
// 0.044715 x^3) ("Kernels, Triton, XLA", section "GeLU three ways: the case
// for fusion"). Since 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), it is evaluated
// as x / (1 + 2^(-2u log2 e)) with the hardware exp2 and reciprocal: no
// branches, finite for every u (exp2 overflow gives -0 for very negative x,
// underflow gives x), a few ulp from the exact value.
__device__ inline float gelu_tanh(float x)
{
    const float u = 0.79788456f * (x + 0.044715f * x * x * x);
    const float e = __builtin_amdgcn_exp2f(u * -2.88539008f);   // exp(-2u); 2.88539008 = 2 log2(e)
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}
template <int ACT>
__device__ inline float activate(float v)
{
    if constexpr (ACT == 0) return __builtin_fmaxf(v, 0.0f);
    else if constexpr (ACT == 1) return gelu_tanh(v);
    else return v;
}
// Runs f(std::integral_constant<int, act>) once: the caller's epilogue is
// compiled once per activation, straight-line, and selected by one uniform
// branch (a test per element would put hundreds of branches in the epilogue).
template <typename F>
__device__ inline void with_activation(int act, F &&f)
{
    if (act == 0) f(std::integral_constant<int, 0>{});
    else if (act == 1) f(std::integral_constant<int, 1>{});
    else f(std::integral_constant<int, 2>{});
}
// Resource over the bias elements of columns n0 .. N-1 (esize bytes each);
// empty (every load reads 0) when there is no bias.
__device__ inline __amdgpu_buffer_rsrc_t make_bias_rsrc(const void *bias, int n0, int N, int esize)
{
    const char *b = static_cast<const char *>(bias);
    const int64_t bytes = b != nullptr ? static_cast<int64_t>(N - n0) * esize : 0;
    return make_store_rsrc(const_cast<char *>(b != nullptr ? b + static_cast<int64_t>(n0) * esize : b), bytes);
}
// Bias of output column n0 + c (c relative to the tile) from a resource over
// the columns n0 .. N-1 of the bias vector; columns past N read 0.
__device__ inline float bias_f32(__amdgpu_buffer_rsrc_t r, int c)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<uint32_t>(c) * 4, 0, 0));
}
__device__ inline float bias_bf16(__amdgpu_buffer_rsrc_t r, int c)
{
    const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<uint32_t>(c) * 2, 0, 0);
    return __uint_as_float(h << 16);
}

__device__ inline void store_b128(__amdgpu_buffer_rsrc_t r, uint32_t voffset, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voffset, 0, 0);
}
__device__ inline void store_b64(__amdgpu_buffer_rsrc_t r, uint32_t voffset, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voffset, 0, 0);
}
__device__ inline void store_b32(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, voffset, 0, 0);
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their "no wait" maxima).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup id -> (tile_m, tile_n). Consecutive workgroup ids go to the 8
// XCDs in turn, each with its own L2, so ids are first regrouped so that each
// XCD owns a contiguous range of logical tiles; that range is then walked in
// bands of `group_m` tile-rows, column by column inside a band, so the tiles
// resident on one XCD at a time share A row-panels and B column-panels.
__device__ inline void tile_of(int64_t id, int64_t grid, int tiles_m, int tiles_n, int group_m,
                               int &tm, int &tn)
{
    constexpr int kXcds = 8;
    int64_t lid = id;
    const int64_t per = grid / kXcds;
    if (per > 0 && id < per * kXcds) lid = (id % kXcds) * per + id / kXcds;
    const int64_t band = static_cast<int64_t>(group_m) * tiles_n;
    const int64_t first_m = (lid / band) * group_m;
    const int64_t rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int64_t in_band = lid % band;
    tm = static_cast<int>(first_m + in_band % rows);
    tn = static_cast<int>(in_band / rows);
}

}  // namespace mmrelu
